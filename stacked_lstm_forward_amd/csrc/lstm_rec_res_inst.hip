// Instantiations of the register-and-LDS resident recurrent kernel for one
// entry of kResShape (selected by LSTM_RES_SHAPE at compile time), with 1 to
// kResMaxNW 16-column batch tiles, without and with the stores of the training
// forward (saved gates, cell and hidden states).
#include "lstm_rec_res.h"

#ifndef LSTM_RES_SHAPE
#error "define LSTM_RES_SHAPE"
#endif

#define LSTM_RES_CAT2(a, b) a##b
#define LSTM_RES_CAT(a, b) LSTM_RES_CAT2(a, b)

namespace lstm {

const void* LSTM_RES_CAT(rec_res_kernel_ptr_shape, LSTM_RES_SHAPE)(int nw, bool save) {
  constexpr ResShape S = kResShape[LSTM_RES_SHAPE];
  constexpr bool BF = S.bf16 != 0;
  const void* const fns[2][kResMaxNW] = {
      {reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 1, S.nci, S.nrb, false>),
       reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 2, S.nci, S.nrb, false>),
       reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 3, S.nci, S.nrb, false>),
       reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 4, S.nci, S.nrb, false>)},
      {reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 1, S.nci, S.nrb, true>),
       reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 2, S.nci, S.nrb, true>),
       reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 3, S.nci, S.nrb, true>),
       reinterpret_cast<const void*>(&lstm_rec_res_kernel<BF, S.mw, 4, S.nci, S.nrb, true>)}};
  static_assert(kResMaxNW == 4, "one instantiation per column-tile count");
  return (nw >= 1 && nw <= kResMaxNW) ? fns[save ? 1 : 0][nw - 1] : nullptr;
}

}  // namespace lstm
