// qmv_variants.hip -- host side of the dense matvec kernels: the variant
// table (its indices are part of the tuning interface), the LDS need of a
// variant, the streaming kernel's occupancy switch and the dispatcher that
// sends a launch to the matrix-core kernel or to its format's vector kernels
// (compiled in separate translation units, one per format).
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

// Variant table.  Indices are part of the tuning interface (qmv_set_tuning).
//   kind, lpr, rows, nu, wpb, ks, xl, name
const Variant kVariants[] = {
    {0, 64, 2, 0, 4, 1, 0, "lpr64_r2"},       {0, 32, 2, 0, 4, 1, 0, "lpr32_r2"},
    {1, 64, 1, 2, 4, 1, 1, "st_w4_r1_u2"},    {1, 64, 2, 2, 4, 1, 1, "st_w4_r2_u2"},
    {1, 64, 1, 3, 4, 1, 1, "st_w4_r1_u3"},    {1, 64, 1, 2, 16, 1, 1, "st_w16_r1_u2"},
    {1, 64, 4, 1, 8, 1, 1, "st_w8_r4_u1"},    {1, 64, 1, 2, 16, 16, 1, "st_k16_r1_u2"},
    {2, 64, 1, 2, 4, 1, 0, "fl_w4_r1_u2_g"},  {2, 64, 2, 2, 4, 1, 0, "fl_w4_r2_u2_g"},
    {2, 64, 1, 3, 4, 1, 0, "fl_w4_r1_u3_g"},  {2, 64, 1, 4, 4, 1, 0, "fl_w4_r1_u4_g"},
    {2, 64, 1, 7, 4, 1, 0, "fl_w4_r1_u7_g"},  {2, 64, 1, 2, 4, 1, 1, "fl_w4_r1_u2_l"},
    {2, 64, 1, 2, 16, 1, 1, "fl_w16_r1_u2_l"}, {2, 64, 1, 3, 16, 1, 1, "fl_w16_r1_u3_l"},
    {2, 64, 1, 7, 8, 1, 1, "fl_w8_r1_u7_l"},  {2, 64, 2, 2, 16, 1, 1, "fl_w16_r2_u2_l"},
    {3, 16, 2, 1, 8, 2, 1, "mt_r2_w8_k2"},    {3, 16, 2, 1, 8, 4, 1, "mt_r2_w8_k4"},
    {3, 16, 4, 1, 8, 2, 1, "mt_r4_w8_k2"},    {3, 16, 4, 1, 4, 1, 1, "mt_r4_w4_k1"},
    {3, 16, 2, 1, 4, 1, 1, "mt_r2_w4_k1"},    {3, 16, 1, 1, 8, 4, 1, "mt_r1_w8_k4"},
    {3, 16, 2, 1, 16, 8, 1, "mt_r2_w16_k8"},  {3, 16, 1, 1, 16, 8, 1, "mt_r1_w16_k8"},
    {3, 16, 2, 2, 8, 2, 1, "mt_r2_u2_w8_k2"}, {3, 16, 2, 2, 8, 1, 1, "mt_r2_u2_w8_k1"},
    {3, 16, 2, 2, 16, 4, 1, "mt_r2_u2_w16_k4"}, {3, 16, 1, 2, 8, 2, 1, "mt_r1_u2_w8_k2"},
    {3, 16, 2, 4, 8, 2, 1, "mt_r2_u4_w8_k2"}, {3, 16, 2, 2, 4, 1, 1, "mt_r2_u2_w4_k1"},
    {3, 16, 1, 2, 16, 4, 1, "mt_r1_u2_w16_k4"}, {3, 16, 1, 4, 16, 4, 1, "mt_r1_u4_w16_k4"},
    {4, 16, 1, 2, 16, 4, 1, "mx_w16_k4_r2"},  {4, 16, 1, 2, 16, 8, 1, "mx_w16_k8_r2"},
    {4, 16, 1, 2, 16, 16, 1, "mx_w16_k16_r2"}, {4, 16, 1, 4, 8, 1, 1, "mx_w8_k1_r4"},
    {4, 16, 1, 4, 8, 4, 1, "mx_w8_k4_r4"},    {4, 16, 1, 4, 8, 8, 1, "mx_w8_k8_r4"},
    {5, 16, 1, 4, 16, 0, 1, "mf_w16_b4"},     {5, 16, 1, 2, 16, 0, 1, "mf_w16_b2"},
    {5, 16, 1, 4, 8, 0, 1, "mf_w8_b4"},       {5, 16, 1, 8, 8, 0, 1, "mf_w8_b8"},
    {6, 64, 1, 2, 16, 16, 0, "lk_w16_r1_u2"}, {6, 64, 1, 4, 8, 8, 0, "lk_w8_r1_u4"},
    {6, 64, 1, 8, 4, 4, 0, "lk_w4_r1_u8"},    {6, 64, 1, 2, 4, 4, 0, "lk_w4_r1_u2"},
    {6, 64, 2, 2, 16, 16, 0, "lk_w16_r2_u2"},
    {2, 64, 2, 2, 4, 1, 1, "fl_w4_r2_u2_l"},  {2, 64, 4, 2, 4, 1, 0, "fl_w4_r4_u2_g"},
    {2, 64, 4, 2, 4, 1, 1, "fl_w4_r4_u2_l"},  {2, 64, 2, 2, 8, 1, 1, "fl_w8_r2_u2_l"},
    {2, 64, 2, 2, 2, 1, 0, "fl_w2_r2_u2_g"},
};
const int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

static int g_bpc_override = 0;  // tuning: workgroups per CU cap (0 = occupancy)
void set_blocks_per_cu(int v) { g_bpc_override = v; }
int blocks_per_cu() { return g_bpc_override; }

static int g_mx_slices = -1;  // tuning: matrix-core cross-workgroup K slices
void set_mx_slices(int v) { g_mx_slices = v; }
int mx_slices() { return g_mx_slices; }

size_t stream_lds_bytes(const Variant& v, int64_t act_bytes, int tm) {
  if (v.kind >= 3) return 0;  // chunked to fit (kMultiLdsBudget)
  if (v.kind == 2) return v.xl || tm > 4 ? static_cast<size_t>(act_bytes) : 0;
  return static_cast<size_t>(act_bytes + (int64_t)v.ks * v.rows * tm * 4);
}

static int variant_index(const char* name) {
  for (int i = 0; i < kNumVariants; ++i)
    if (__builtin_strcmp(kVariants[i].name, name) == 0) return i;
  return 0;
}

hipError_t launch_matvec(const MatvecLaunch& a, hipStream_t st) {
  const Variant& v = kVariants[a.variant];
  if (v.kind == 5) {
    // the flat matrix-core kernel, split over workgroups only with a
    // workspace; without a plan that fits (or for a batched launch) the
    // persistent matrix-core kernel of the same workgroup size
    MxfPlan p{};
    const bool can_split = a.part != nullptr && a.cnt != nullptr && mx_slices() != 0;
    if (a.seg.n == 0 &&
        mxf_plan(a.fmt, a.n_tok, v.wpb, v.nu, a.units, a.n_rows, a.cus, a.lds_per_cu, can_split,
                 mx_slices() >= 2 ? mx_slices() : 0, &p) > 0)
      return launch_mxf(a, p, st);
    MatvecLaunch b = a;
    b.variant = variant_index(v.wpb == 16 ? "mx_w16_k4_r2" : "mx_w8_k4_r4");
    return launch_mx(b, st);
  }
  if (v.kind == 4) return launch_mx(a, st);
  switch (a.fmt) {
    case FQ8_0: return launch_vector<FQ8_0>(a, st);
    case FQ4_K: return launch_vector<FQ4_K>(a, st);
    case FIQ4_XS: return launch_vector<FIQ4_XS>(a, st);
    case FQ5_K: return launch_vector<FQ5_K>(a, st);
    case FQ6_K: return launch_vector<FQ6_K>(a, st);
    case FQ8G128: return launch_vector<FQ8G128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmv
