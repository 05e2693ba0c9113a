// Instantiations of the register-and-LDS resident recurrent kernel for one
// entry of kResShape (selected by LSTM_RES_SHAPE at compile time), with 1 to
// kResMaxNW 16-column batch tiles.
#include "lstm_rec_res.h"

#ifndef LSTM_RES_SHAPE
#error "define LSTM_RES_SHAPE"
#endif

#define LSTM_RES_CAT2(a, b) a##b
#define LSTM_RES_CAT(a, b) LSTM_RES_CAT2(a, b)

namespace lstm {

const void* LSTM_RES_CAT(rec_res_kernel_ptr_shape, LSTM_RES_SHAPE)(int nw) {
  constexpr ResShape S = kResShape[LSTM_RES_SHAPE];
  switch (nw) {
    case 1:
      return reinterpret_cast<const void*>(&lstm_rec_res_kernel<S.bf16 != 0, S.mw, 1, S.nci, S.nrb>);
    case 2:
      return reinterpret_cast<const void*>(&lstm_rec_res_kernel<S.bf16 != 0, S.mw, 2, S.nci, S.nrb>);
    case 3:
      return reinterpret_cast<const void*>(&lstm_rec_res_kernel<S.bf16 != 0, S.mw, 3, S.nci, S.nrb>);
    case 4:
      return reinterpret_cast<const void*>(&lstm_rec_res_kernel<S.bf16 != 0, S.mw, 4, S.nci, S.nrb>);
  }
  return nullptr;
}

}  // namespace lstm
