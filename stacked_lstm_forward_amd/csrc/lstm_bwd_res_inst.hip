// Instantiations of the backward pass's on-chip chain kernel for one entry of
// kBwdResShape (selected by LSTM_BWD_RES_SHAPE at compile time), with 1, 2 and
// 4 16-column batch tiles (2 at most for four M-tiles with NCI = 16, whose
// registers hold 48 weight blocks).
#include "lstm_bwd_res.h"

#ifndef LSTM_BWD_RES_SHAPE
#error "define LSTM_BWD_RES_SHAPE"
#endif

#define LSTM_BWD_RES_CAT2(a, b) a##b
#define LSTM_BWD_RES_CAT(a, b) LSTM_BWD_RES_CAT2(a, b)

namespace lstm {

const void* LSTM_BWD_RES_CAT(bwd_res_kernel_ptr_shape, LSTM_BWD_RES_SHAPE)(int nw) {
  constexpr BwdResShape S = kBwdResShape[LSTM_BWD_RES_SHAPE];
  constexpr bool BF = S.bf16 != 0;
  if (nw == 1) return reinterpret_cast<const void*>(&lstm_bwd_res_kernel<BF, 1, S.nci, S.mw>);
  if (nw == 2) return reinterpret_cast<const void*>(&lstm_bwd_res_kernel<BF, 2, S.nci, S.mw>);
  if constexpr (S.mw == 1 || S.nci < 16) {
    if (nw == 4) return reinterpret_cast<const void*>(&lstm_bwd_res_kernel<BF, 4, S.nci, S.mw>);
  }
  return nullptr;
}

}  // namespace lstm
