// Instantiations of the persistent recurrent kernel for one (dtype, weight
// source) pair, selected by LSTM_INST_BF16 / LSTM_INST_STREAM at compile time:
// the aligned fast path for every tile shape MW x NW in {1, 2, 4}^2, and the
// ragged-size path at the largest shape (4 x 4), which covers every plan.
#include "lstm_rec.h"

#ifndef LSTM_INST_BF16
#error "define LSTM_INST_BF16"
#endif
#ifndef LSTM_INST_STREAM
#error "define LSTM_INST_STREAM"
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
#define LSTM_CAT3(a, b, c) a##b##_##c
#define LSTM_FN_NAME(d, s) LSTM_CAT3(rec_kernel_ptr_, d, s)

namespace lstm {

const void* LSTM_FN_NAME(LSTM_DT_NAME, LSTM_SRC_NAME)(int mw, int nw, bool vec) {
  constexpr bool BF = LSTM_INST_BF16 != 0;
  constexpr bool ST = LSTM_INST_STREAM != 0;
  if (!vec) return reinterpret_cast<const void*>(&lstm_rec_kernel<BF, 4, 4, ST, false>);
  const int MW = mw <= 1 ? 1 : (mw <= 2 ? 2 : 4);
  const int NW = nw <= 1 ? 1 : (nw <= 2 ? 2 : 4);
#define LSTM_REC_CASE(M, N) \
  if (MW == M && NW == N) return reinterpret_cast<const void*>(&lstm_rec_kernel<BF, M, N, ST, true>);
  LSTM_REC_CASE(1, 1) LSTM_REC_CASE(1, 2) LSTM_REC_CASE(1, 4)
  LSTM_REC_CASE(2, 1) LSTM_REC_CASE(2, 2) LSTM_REC_CASE(2, 4)
  LSTM_REC_CASE(4, 1) LSTM_REC_CASE(4, 2) LSTM_REC_CASE(4, 4)
#undef LSTM_REC_CASE
  return nullptr;
}

}  // namespace lstm
