// Randomised problem descriptions through the host planner (make_plan,
// data_valid_lds), built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_planner_sanitized.py.  Besides running clean under the
// sanitizers, every accepted plan must satisfy the invariants the launch code
// relies on; a violation prints the description and exits with status 1.
#include <cstdio>
#include <cstdlib>
#include <cstdint>

#include "lstm_plan.h"

using namespace lstm;

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int pick(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }
int pick_dim() {  // small, aligned, ragged and large values
  static const int fixed[] = {1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129,
                              255, 256, 257, 511, 512, 513, 1000, 1023, 1024, 1536, 2048, 3000, 4096, 6144, 8192};
  if (next_u64() % 4 == 0) return pick(1, 9000);
  return fixed[next_u64() % (sizeof(fixed) / sizeof(fixed[0]))];
}

int fail(const char* what, int L, int I, int H, int B, int T, int dt, int cell, int force) {
  std::printf("invariant failed: %s  (L=%d I=%d H=%d B=%d T=%d dtype=%d cell=%d regime=%d)\n", what, L, I, H, B, T,
              dt, cell, force);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 20000;
  if (argc > 2) g_state = std::strtoull(argv[2], nullptr, 10);
  int accepted = 0;
  for (int it = 0; it < n; ++it) {
    const int L = next_u64() % 8 == 0 ? pick(1, 70) : pick(1, 6);
    const int I = pick_dim(), H = pick_dim(), B = next_u64() % 6 == 0 ? pick(1, 300) : pick(1, 80);
    const int T = pick(1, 300), dt = pick(0, 1), cell = pick(0, 3), force = pick(0, 2);
    DeviceInfo dev;
    dev.num_cus = next_u64() % 5 == 0 ? pick(1, 304) : 256;
    dev.lds_per_block = next_u64() % 7 == 0 ? 64 * 1024 : 160 * 1024;
    Plan p;
    const bool aligned = next_u64() % 3 != 0;
    const int rc = make_plan(L, I, H, B, T, dt, cell, force, dev, &p, aligned);
    if (rc != 0) continue;
    ++accepted;
    if (p.nrec < 1 || p.nrec > 64) return fail("launch count", L, I, H, B, T, dt, cell, force);
    if (p.ws_bytes < p.hist_off || p.hist_off < p.G_off || p.G_off < p.flags_off)
      return fail("workspace layout order", L, I, H, B, T, dt, cell, force);
    if (p.slot_elems * (size_t)p.dsize < (size_t)B * H * p.dsize)
      return fail("exchange slot too small", L, I, H, B, T, dt, cell, force);
    int layers = 0;
    for (int r = 0; r < p.nrec; ++r) {
      const LaunchPlan& lp = p.rec[r];
      if (lp.nlayers < 1 || lp.nlayers > kMaxLayersPerLaunch) return fail("layers per launch", L, I, H, B, T, dt, cell, force);
      if (lp.grid < 1 || lp.grid > (dev.num_cus > 8 ? dev.num_cus : 8)) return fail("grid", L, I, H, B, T, dt, cell, force);
      if (lp.lds_bytes + 256 > dev.lds_per_block) return fail("LDS", L, I, H, B, T, dt, cell, force);
      if (lp.nwaves != 4 && lp.nwaves != 8) return fail("waves", L, I, H, B, T, dt, cell, force);
      if (lp.ks < 1 || lp.ks > lp.nwaves || lp.nwaves % lp.ks) return fail("K split", L, I, H, B, T, dt, cell, force);
      if (lp.ntgm * lp.ntgn * lp.ks != lp.nwaves) return fail("tile groups", L, I, H, B, T, dt, cell, force);
      int wgs = 0, mts = 0;
      for (int k = 0; k < lp.nlayers; ++k) {
        const LayerPlan& pl = lp.layers[k];
        if (pl.wg_begin != wgs) return fail("workgroup ranges", L, I, H, B, T, dt, cell, force);
        if (pl.wg_count < 1 || pl.wg_count > kFlagsPerLayer) return fail("workgroups per layer", L, I, H, B, T, dt, cell, force);
        if (pl.mt_per_wg < 1 || pl.mt_per_wg > 16) return fail("M-tiles per workgroup", L, I, H, B, T, dt, cell, force);
        if ((long)pl.wg_count * pl.mt_per_wg < p.Mt) return fail("M-tiles covered", L, I, H, B, T, dt, cell, force);
        wgs += pl.wg_count;
        mts += pl.mt_per_wg;
        ++layers;
      }
      if (wgs > lp.grid) return fail("grid holds the workgroups", L, I, H, B, T, dt, cell, force);
      (void)mts;
      const int dv = data_valid_lds(p, lp, H, B, dev);
      if (dv < 0 || dv + 256 > dev.lds_per_block) return fail("data-valid LDS", L, I, H, B, T, dt, cell, force);
    }
    if (layers != L) return fail("every layer planned once", L, I, H, B, T, dt, cell, force);
  }
  std::printf("ok: %d of %d descriptions accepted\n", accepted, n);
  return 0;
}
