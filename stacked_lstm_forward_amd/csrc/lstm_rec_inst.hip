// Instantiations of the persistent recurrent kernel for one (dtype, weight
// source, waves per workgroup) triple, selected by LSTM_INST_BF16 /
// LSTM_INST_STREAM / LSTM_INST_NWV at compile time:
// the aligned fast path for every tile shape MW x NW in {1, 2, 4}^2, with the
// row-major and the load-order exchange, and the ragged-size path (row-major)
// at the largest shape (4 x 4), which covers every plan.
// Workgroups of 8 waves are planned with at most 4 tiles per wave (larger tile
// sets spill at two waves per SIMD), so they need only the shapes with
// MW*NW <= 4 and their ragged path comes in the three covering shapes.
#include "lstm_rec.h"

#ifndef LSTM_INST_BF16
#error "define LSTM_INST_BF16"
#endif
#ifndef LSTM_INST_STREAM
#error "define LSTM_INST_STREAM"
#endif
#ifndef LSTM_INST_NWV
#error "define LSTM_INST_NWV"
#endif

#if LSTM_INST_BF16
#define LSTM_DT_NAME bf16
#else
#define LSTM_DT_NAME f32
#endif
#if LSTM_INST_STREAM
#define LSTM_SRC_NAME stream
#else
#define LSTM_SRC_NAME lds
#endif
#define LSTM_CAT4(a, b, c, w) a##b##_##c##_w##w
#define LSTM_FN_NAME(d, s, w) LSTM_CAT4(rec_kernel_ptr_, d, s, w)

namespace lstm {

const void* LSTM_FN_NAME(LSTM_DT_NAME, LSTM_SRC_NAME, LSTM_INST_NWV)(int mw, int nw, bool vec, bool frag) {
  constexpr bool BF = LSTM_INST_BF16 != 0;
  constexpr bool ST = LSTM_INST_STREAM != 0;
  constexpr int NV = LSTM_INST_NWV;
#if LSTM_INST_NWV == 8
  if (mw * nw > 4) return nullptr;
  if (!vec) {
    if (frag) return nullptr;
    if (nw == 1) return reinterpret_cast<const void*>(&lstm_rec_kernel<BF, 4, 1, ST, false, NV, false>);
    if (mw == 1) return reinterpret_cast<const void*>(&lstm_rec_kernel<BF, 1, 4, ST, false, NV, false>);
    return reinterpret_cast<const void*>(&lstm_rec_kernel<BF, 2, 2, ST, false, NV, false>);
  }
#else
  if (!vec) return frag ? nullptr : reinterpret_cast<const void*>(&lstm_rec_kernel<BF, 4, 4, ST, false, NV, false>);
#endif
  const int MW = mw <= 1 ? 1 : (mw <= 2 ? 2 : 4);
  const int NW = nw <= 1 ? 1 : (nw <= 2 ? 2 : 4);
#define LSTM_REC_CASE(M, N)                                                                                  \
  if (MW == M && NW == N)                                                                                    \
    return frag ? reinterpret_cast<const void*>(&lstm_rec_kernel<BF, M, N, ST, true, NV, true>)             \
                : reinterpret_cast<const void*>(&lstm_rec_kernel<BF, M, N, ST, true, NV, false>);
  LSTM_REC_CASE(1, 1) LSTM_REC_CASE(1, 2) LSTM_REC_CASE(1, 4)
  LSTM_REC_CASE(2, 1) LSTM_REC_CASE(2, 2) LSTM_REC_CASE(4, 1)
#if LSTM_INST_NWV != 8
  LSTM_REC_CASE(2, 4) LSTM_REC_CASE(4, 2) LSTM_REC_CASE(4, 4)
#endif
#undef LSTM_REC_CASE
  return nullptr;
}

}  // namespace lstm
