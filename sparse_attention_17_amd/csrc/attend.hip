// Host dispatch of the core attention (CSA: selected compressed entries +
// sliding window + sink; HCA: every completed m'-block + optional window +
// sink).  The kernels are templates in attend_impl.hpp, instantiated per
// variant in the attend_v_*.hip translation units.
#include "attend_impl.hpp"

namespace csa {

// instantiated in the attend_v_*.hip translation units
extern template hipError_t attend_variant<float, 64, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
extern template hipError_t attend_variant<float, 128, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
extern template hipError_t attend_variant<bf16, 64, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
extern template hipError_t attend_variant<bf16, 128, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
extern template hipError_t attend_variant<bf16, 128, true>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
extern template hipError_t pair_variant<float, 64>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
extern template hipError_t combine_pair_variant<float, 64>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);
extern template hipError_t pair_variant<float, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
extern template hipError_t combine_pair_variant<float, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);
extern template hipError_t pair_variant<bf16, 64>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
extern template hipError_t combine_pair_variant<bf16, 64>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);
extern template hipError_t pair_variant<bf16, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
extern template hipError_t combine_pair_variant<bf16, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);

size_t attend_workspace(bool sparse, int B, int Tq, int H, int d, int topk, int window,
                        int Nc_cap, int m_prime, int max_pos) {
  const long nk = nkeys_upper(sparse, topk, window, Nc_cap, m_prime, max_pos);
  const int kps = keys_per_split(sparse, Tq, nk);
  const long ns = std::max(1L, (nk + kps - 1) / kps);
  if (ns <= 1) return 0;
  return (size_t)ns * B * Tq * H * (d + 2) * sizeof(float);
}

static hipError_t dispatch(const AttendArgs& a, const AttnGeom& gm, const AttendLaunch& how, hipStream_t st) {
  if (a.kv8) return a.d == 128 && !a.f32 ? attend_variant<bf16, 128, true>(a, gm, how, st) : hipErrorInvalidValue;
  if (a.f32) return a.d == 64 ? attend_variant<float, 64, false>(a, gm, how, st)
                              : attend_variant<float, 128, false>(a, gm, how, st);
  return a.d == 64 ? attend_variant<bf16, 64, false>(a, gm, how, st)
                   : attend_variant<bf16, 128, false>(a, gm, how, st);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  if (a.B == 0 || a.Tq == 0) return hipSuccess;
  return dispatch(a, make_geom(a), AttendLaunch{}, st);
}

static hipError_t combine_pair(const AttendArgs& h, const AttnGeom& gh, const AttendArgs& c,
                               const AttnGeom& gc, hipStream_t st) {
  if (c.f32) return c.d == 64 ? combine_pair_variant<float, 64>(h, gh, c, gc, st)
                              : combine_pair_variant<float, 128>(h, gh, c, gc, st);
  return c.d == 64 ? combine_pair_variant<bf16, 64>(h, gh, c, gc, st)
                   : combine_pair_variant<bf16, 128>(h, gh, c, gc, st);
}

hipError_t launch_attend_pair(const AttendArgs& csa_a, const AttendArgs& hca_a, hipStream_t st) {
  if (csa_a.B == 0 || csa_a.Tq == 0) return launch_attend(hca_a, st);
  if (hca_a.B == 0 || hca_a.Tq == 0) return launch_attend(csa_a, st);
  const AttnGeom gc = make_geom(csa_a), gh = make_geom(hca_a);
  int rwc, kgc, rwh, kgh;
  wave_shape(gc.TT * csa_a.H, &rwc, &kgc);
  wave_shape(gh.TT * hca_a.H, &rwh, &kgh);
  // one launch needs the same kernel shape for both (split decode, same
  // element type, head dim and wave layout); otherwise they run one after the other
  const bool fuse = gc.nsplit > 1 && gh.nsplit > 1 && csa_a.f32 == hca_a.f32 && csa_a.d == hca_a.d &&
                    rwc == rwh && kgc == kgh && !csa_a.kv8 && !hca_a.kv8;
  if (!fuse) {
    const hipError_t e = launch_attend(csa_a, st);
    return e != hipSuccess ? e : launch_attend(hca_a, st);
  }
  if (csa_a.f32)
    return csa_a.d == 64 ? pair_variant<float, 64>(hca_a, gh, csa_a, gc, rwc, st)
                         : pair_variant<float, 128>(hca_a, gh, csa_a, gc, rwc, st);
  return csa_a.d == 64 ? pair_variant<bf16, 64>(hca_a, gh, csa_a, gc, rwc, st)
                       : pair_variant<bf16, 128>(hca_a, gh, csa_a, gc, rwc, st);
}

}  // namespace csa
