// Instantiations of the register-and-LDS resident recurrent kernel: bf16,
// kResMW = 4 M-tiles per workgroup, kResNCI = 16 chunks of 64 columns per
// K-group (H = 4096), one or two 16-column batch tiles; kResNRB = 48 of a
// wave's 64 blocks stay in registers (384 of its 512), the other 16 per wave
// (128 KiB per workgroup) in LDS.
#include "lstm_rec_res.h"

namespace lstm {

const void* rec_res_kernel_ptr(bool bf16, int mw, int nw, int nci, int nrb) {
  if (!bf16 || mw != kResMW || nci != kResNCI || nrb != kResNRB) return nullptr;
  if (nw == 1) return reinterpret_cast<const void*>(&lstm_rec_res_kernel<true, kResMW, 1, kResNCI, kResNRB>);
  if (nw == 2) return reinterpret_cast<const void*>(&lstm_rec_res_kernel<true, kResMW, 2, kResNCI, kResNRB>);
  return nullptr;
}

}  // namespace lstm
