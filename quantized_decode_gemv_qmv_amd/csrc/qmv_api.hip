// qmv_api.hip -- host side of the C ABI declared in include/qmv.h:
// argument validation (before anything is enqueued), kernel-variant and
// split-K choice, workspace layout, size queries and status strings.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "qmv_internal.h"
#include "qmv_mfma.h"
#include "qmv.h"

#define QMV_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace qmv;

constexpr int64_t kSplitMaxRows = 8192;   // split-K only for few-row shapes
constexpr int64_t kMoeMaxUnits = 512;     // k <= 16384 for the MoE kernel

std::atomic<int64_t> g_splitk{-1};
// The flat kernel's split over workgroups is off by default: its cross-
// workgroup handoff adds a few microseconds at the end of kernels that take
// 5-10 us (256 x 65536 Q8_0, one token: 10.3 us split, 7.4 us for the
// streaming kernel's in-workgroup split), and the variant choice above
// avoids the shapes where it won.
std::atomic<int64_t> g_flat_split{0};
bool flat_split_enabled() { return g_flat_split.load() != 0; }
std::atomic<int64_t> g_variant{-1};
// Fused MoE gate+up + SwiGLU kernel: -1 automatic, 0 never, 1 always (where it applies).
std::atomic<int64_t> g_ffn_fuse{-1};

struct EnvInit {
  EnvInit() {
    if (const char* v = std::getenv("QMV_SPLITK")) {
      if (!std::strcmp(v, "auto")) g_splitk = -1;
      else if (!std::strcmp(v, "off")) g_splitk = 0;
      else g_splitk = std::atoll(v);
    }
    if (const char* v = std::getenv("QMV_VARIANT")) g_variant = std::atoll(v);
    if (const char* v = std::getenv("QMV_MOE_KERNEL")) {
      const int k = std::atoi(v);
      if (k >= 0 && k <= 3) set_moe_kernel(k);
    }
  }
} g_env_init;

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

bool valid_type(int t) {
  return t == QMV_Q8_0 || t == QMV_Q4_K || t == QMV_IQ4_XS || t == QMV_Q5_K || t == QMV_Q6_K || t == QMV_Q8G128;
}

int64_t block_k(int t) { return t == QMV_Q8_0 ? 32 : (t == QMV_Q8G128 ? 128 : 256); }
int64_t block_bytes(int t) {
  switch (t) {
    case QMV_Q8_0: return 34;
    case QMV_Q4_K: return 144;
    case QMV_IQ4_XS: return 136;
    case QMV_Q5_K: return 176;
    case QMV_Q8G128: return 130;
    default: return 210;  // q6_K
  }
}
// Formats the matrix-core kernels and the MoE kernels decode.
// Formats with a matrix-core decode (dense kernels), and those the
// expert-grouped MoE kernels take.
bool has_mfma(int t) { return t == QMV_Q8_0 || t == QMV_Q4_K || t == QMV_IQ4_XS || t == QMV_Q8G128; }
bool moe_format(int t) { return t == QMV_Q8_0 || t == QMV_Q4_K || t == QMV_IQ4_XS; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct DeviceInfo {
  int cus;
  int64_t lds_per_cu;
  int64_t lds_per_block;
};

// Properties of the current device, queried once per device.  Without a
// device (host-only size and plan queries) and for attributes the runtime
// does not report, those of the MI355X (gfx950) the library is built for:
// 256 compute units, 160 KiB of LDS per compute unit and per workgroup.
constexpr int kDefaultCus = 256;
constexpr int64_t kDefaultLds = 160 * 1024;
DeviceInfo device_info() {
  static std::mutex mu;
  static DeviceInfo cache[64];
  static bool have[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return {kDefaultCus, kDefaultLds, kDefaultLds};
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    int cus = 0, lcu = 0, lblk = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = kDefaultCus;
    if (hipDeviceGetAttribute(&lcu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        lcu <= 0)
      lcu = kDefaultLds;
    if (hipDeviceGetAttribute(&lblk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        lblk <= 0)
      lblk = kDefaultLds;
    cache[dev] = {cus, lcu, lblk};
    have[dev] = true;
  }
  return cache[dev];
}

int device_cus() { return device_info().cus; }

ActView act_view(const void* xq, int64_t n_tok, int64_t k) {
  const uint8_t* b = static_cast<const uint8_t*>(xq);
  ActView v;
  v.qs = reinterpret_cast<const int8_t*>(b);
  v.d = reinterpret_cast<const float*>(b + qmv_act_offset_d(n_tok, k));
  v.s = reinterpret_cast<const int32_t*>(b + qmv_act_offset_s(n_tok, k));
  v.k = static_cast<int>(k);
  v.nb = static_cast<int>(k / 32);
  return v;
}

qmv_status check_weights(int type, const void* w, int64_t n_rows, int64_t k) {
  if (!valid_type(type) || w == nullptr || n_rows < 1 || k < 1 || k % block_k(type) != 0)
    return QMV_ERR_INVALID_ARG;
  if (n_rows > INT32_MAX / 4 || k / 32 > INT32_MAX / 64) return QMV_ERR_INVALID_ARG;
  if (!aligned(w, 16)) return QMV_ERR_MISALIGNED;
  return QMV_OK;
}

int find_variant(const char* name) {
  for (int i = 0; i < kNumVariants; ++i)
    if (!std::strcmp(kVariants[i].name, name)) return i;
  return 0;
}

int token_capacity(int64_t n_tok) {
  return n_tok <= 1 ? 1 : n_tok <= 2 ? 2 : n_tok <= 4 ? 4 : n_tok <= 8 ? 8 : 16;
}

// Whether a streaming variant's LDS staging fits one workgroup.
bool stream_fits(int v, int64_t k, int64_t n_tok) {
  const Variant& var = kVariants[v];
  if (var.kind == 0) return true;
  const size_t need =
      stream_lds_bytes(var, (int64_t)qmv_act_bytes(n_tok, k), token_capacity(n_tok));
  return (int64_t)need <= device_info().lds_per_block;
}

// Default kernel for a shape, from measurements on MI355X of every variant on
// the workload shapes (Q8_0 4096x4096, 14336x4096 and 152064x5120, q4_K,
// q5_K and q6_K 14336x4096, IQ4_XS 4096x14336, Q8_0 256x65536, Q8G128
// 152064x5120, 14336x4096, 4096x4096 and 4096x14336; 1..16 tokens):
//   - up to 1024 rows of at least 256 blocks, up to four tokens: the
//     long-row kernel (a workgroup's waves split one row's K, activation
//     fragments from global memory), the flat kernel on 1024 rows from three
//     tokens;
//   - up to two tokens (four for Q8_0): the flat kernel (one wave per row
//     group, all loads issued at once), its units per lane sized so that one
//     chunk covers the row;
//   - 3..8 tokens: the matrix-core kernel for IQ4_XS (and q4_K from five
//     tokens), 16-wave workgroups with K split so that about 4096 waves
//     cover the rows; otherwise the multi-token vector kernel;
//   - 9..16 tokens: the matrix-core kernel (for Q8_0 and Q8G128 only from
//     128 rows per compute unit), 8-wave workgroups with a four-deep load ring (the
//     register budget of the 16-token tiles);
//   - q5_K and q6_K have no matrix-core decode: from three tokens the
//     multi-token vector kernel (q5_K, and q6_K on long rows) or the flat
//     one (q6_K while one chunk of 128 units per lane covers the row);
//   - Q8_0 at 5..8 tokens, Q8G128 at 3..8 (and both from nine on fewer
//     than 128 rows per compute unit): by rows per compute unit, the flat kernel with 16-wave
//     workgroups on many rows (on rows of more than 128 blocks only up to
//     four tokens, the multi-token one from five), the
//     multi-token kernel with two rows per lane group in between, and the
//     flat kernel (or, on long rows from nine tokens, the multi-token one
//     splitting K four ways) on few rows.
//   The vector multi-token kernel's LDS staging is chunked and so fits any
//   K, which also makes it the fallback.
int auto_variant(int type, int64_t n_rows, int64_t k, int64_t n_tok) {
  const int64_t units = k / 32;
  const int cus = device_cus();
  const int64_t nu = (units + 63) / 64;
  const int64_t rpc = n_rows / cus;  // rows per compute unit
  const int64_t tiles = (n_rows + 15) / 16;
  const char* name;
  if (n_rows <= 4 * (int64_t)cus && units >= 256 && n_tok <= 4) {
    // few rows, long K: the long-row kernel, a workgroup's waves splitting
    // the K of one row with activation fragments from global memory
    // (measured at 1 / 2 / 4 tokens, us: Q8_0 256 x 65536 6.09 / 6.75 / 8.95
    // against 7.29 for the LDS-staged streaming kernel and 20.38 / 25.02 for
    // the flat one (the streaming staging does not fit from two tokens);
    // q4_K 256 x 65536 4.80 / 5.81 / 8.10 against 6.11 / 13.58 / 15.51;
    // 512 x 16384 Q8_0 4.08 / 4.58 / 5.67, IQ4_XS 3.57 / 4.13 / 5.19 against
    // 5.42 / 6.42 / 7.49 and 4.94 / 5.07 / 6.78 for the flat kernel): eight
    // waves of four units per lane up to one row per compute unit and two
    // tokens (sixteen of two units at three and four, and at one for Q8_0
    // and for q4_K rows of up to 32768 weights: 5.84 against 6.10 us on Q8_0
    // 256 x 65536, 3.64 against 3.83 on q4_K 256 x 32768), four of two units up
    // to two rows per compute unit; on 1024 rows (IQ4_XS x 8192) the same up
    // to two tokens (3.40 / 3.78 us against 3.44 / 3.86) and the flat kernel
    // from three (4.60 against 4.76 us at four)
    if (n_rows <= cus)
      name = n_tok <= 2 && !(n_tok == 1 && (type == QMV_Q8_0 || (type == QMV_Q4_K && units <= 1024)))
                 ? "lk_w8_r1_u4"
                 : "lk_w16_r1_u2";
    else
      name = n_rows <= 2 * (int64_t)cus || n_tok <= 2 ? "lk_w4_r1_u2" : "fl_w4_r1_u4_g";
  } else if (n_rows < 4 * (int64_t)cus && units >= 256) {
    // the same shapes at more tokens: where the streaming kernel's staging
    // does not fit, the matrix-core kernel (q4_K 256 x 65536 at four tokens:
    // 15.8 us against 46 us for the multi-token vector kernel)
    name = stream_fits(find_variant("st_k16_r1_u2"), k, n_tok) ? "st_k16_r1_u2"
           : has_mfma(type)                                     ? "mx_w8_k8_r4"
                                                                : "mt_r2_w8_k4";
  } else if ((type == QMV_Q4_K || type == QMV_IQ4_XS) && nu <= 2 && n_tok <= 16 && rpc >= 16 &&
             (n_tok > 2 || rpc == 16 || type == QMV_Q4_K)) {
    // q4_K and IQ4_XS rows of up to 4096 weights (measured on 4096, 8192 and
    // 14336 rows x 4096, us at 16 / 32 / 56 rows per compute unit):
    //  - up to 3 tokens the flat kernel, one row per wave on 16 rows per
    //    compute unit (IQ4_XS at 3 tokens 5.04 against 8.30 for the
    //    matrix-core kernel, q4_K 5.23 against 5.39 with two rows), else two;
    //  - 4 tokens eight waves of two rows below 48 rows per compute unit
    //    (IQ4_XS 8192 rows 7.51 against 10.09, q4_K 7.79 against 8.17);
    //  - 5..8 tokens the same below 24 rows per compute unit (IQ4_XS 6.80 at
    //    5 against 8.56), the flat matrix-core kernel from there (IQ4_XS
    //    14336 rows 13.3 against 14.0, 8192 rows 9.6 against 10.6);
    //  - 9..16 tokens the flat matrix-core kernel below 48 rows per compute
    //    unit (8192 rows at 16 tokens: q4_K 9.84 against 12.52, IQ4_XS 10.92
    //    against 13.25; IQ4_XS keeps the persistent one on 16 rows, 9.98
    //    against 10.32), then the persistent one (IQ4_XS with 16-wave
    //    workgroups: 15.37 against 16.36 at 16 tokens on 14336 rows).
    //  - from 96 rows per compute unit (28672 x 4096) the persistent
    //    matrix-core kernel with one wave per row tile from 5 tokens (q4_K /
    //    IQ4_XS at 6 tokens 20.0 / 20.5 us against 22.4 / 24.2 for the flat
    //    one, at 16 tokens 22.3 / 23.6 against 23.0 / 25.8), eight waves of
    //    two rows at 4 (IQ4_XS 19.3 against 20.5).
    const bool q4k = type == QMV_Q4_K;
    if (rpc >= 96 && n_tok >= 4)
      name = n_tok == 4 ? "fl_w8_r2_u2_l" : "mx_w8_k1_r4";
    else if (n_tok <= 3)
      name = rpc == 16 ? "fl_w4_r1_u2_l" : q4k || n_tok == 3 ? "fl_w4_r2_u2_l" : "fl_w4_r2_u2_g";
    else if (n_tok == 4)
      name = rpc < 48 ? "fl_w8_r2_u2_l" : "fl_w4_r2_u2_l";
    else if (n_tok <= 8)
      name = rpc < 24 ? "fl_w8_r2_u2_l" : "mf_w8_b4";
    else
      name = rpc < 24 && !q4k ? "mx_w8_k8_r4" : rpc < 48 ? "mf_w8_b4" : q4k ? "mx_w8_k4_r4" : "mx_w16_k4_r2";
  } else if ((type == QMV_Q5_K || type == QMV_Q6_K) && n_tok <= 16 && rpc >= 16 && (nu <= 2 || rpc <= 24)) {
    // q5_K and q6_K (vector kernels only), measured on 4096 / 8192 / 14336
    // x 4096 and 4096 x 14336 (us):
    //  - rows of more than 128 blocks (16 rows per compute unit): at one
    //    token four waves of two units per lane (q5_K one row per wave
    //    10.48, q6_K two 14.57, against 11.50 / 17.45 with seven units), at
    //    2..8 tokens sixteen waves of one row (q6_K at 4 18.20 against 29.71
    //    for the multi-token kernel; q5_K keeps seven units at 2), from 9 the
    //    multi-token kernel with eight waves splitting K four ways (q6_K at
    //    16 45.28 against 132.86 with two);
    //  - rows of up to 128 blocks: two and three tokens (and four for
    //    q6_K) one row per wave on 16 rows per compute unit, else two (q6_K
    //    4096 x 4096 at 3 6.38 against 6.86); q5_K at 4 as q4_K, from 5
    //    the multi-token kernel, one row per lane group and K split four
    //    ways on 16 rows per compute unit (11.81 against 26.81 at 16
    //    tokens), two rows below 48 (18.24 against 27.59), four from 9
    //    tokens above; q6_K from 5 as measured on 14336 x 4096 (below).
    const bool q6 = type == QMV_Q6_K;
    if (nu > 2)
      name = n_tok == 1                ? (q6 ? "fl_w4_r2_u2_l" : "fl_w4_r1_u2_l")
             : n_tok == 2 && !q6       ? "fl_w8_r1_u7_l"
             : n_tok <= 8              ? "fl_w16_r1_u2_l"
                                       : "mt_r1_w8_k4";
    else if (n_tok == 1)
      name = "fl_w4_r2_u2_g";
    else if (n_tok <= 3 || (q6 && n_tok == 4))
      name = rpc == 16 ? "fl_w4_r1_u2_l" : "fl_w4_r2_u2_l";
    else if (!q6 && n_tok == 4)
      name = rpc < 48 ? "fl_w8_r2_u2_l" : "fl_w4_r2_u2_l";
    else if (q6)
      name = n_tok == 5 || (n_tok >= 9 && n_tok <= 10) ? "fl_w4_r2_u2_g" : "fl_w8_r2_u2_l";
    else
      name = rpc < 24 ? "mt_r1_w8_k4" : rpc < 48 || n_tok <= 8 ? "mt_r2_w8_k2" : "mt_r4_w8_k2";
  } else if (type == QMV_Q8G128 && n_tok == 2 && rpc >= 128) {
    name = "st_w4_r1_u3";  // the head at two tokens: 144.0 / 142.0 us against 151.0 / 150.4 (two boxes)
  } else if (n_tok <= (type == QMV_Q8_0 ? 4 : 2) ||
             (type == QMV_Q4_K && n_tok <= 4 && nu <= 2 && n_rows >= 8 * (int64_t)cus)) {
    // q4_K 14336 x 4096 at 1 / 2 / 3 / 4 tokens: two rows per wave with the
    // activations staged in LDS 7.75 / 8.43 / 10.34 / 11.07 us, with
    // fragments from global memory 7.80 / 8.97 / 12.51 / 12.57, the flat
    // matrix-core kernel 11.9 at 3 and 4 (medians; at 5..8 tokens the flat
    // kernel's eight-token instantiation takes 16.5 us and more).  Q8_0
    // 4096 x 4096 at four tokens: eight waves of two rows 6.07 against 6.39
    // for one row per wave.
    // Q8_0 at four tokens on up to 64 rows per compute unit: eight waves of
    // two rows (4096 / 8192 / 14336 x 4096: 6.11 / 9.13 / 14.44 us against
    // 6.38 / 9.84 / 15.20 for one row per wave); rows of 14336 weights on 16
    // rows per compute unit at two to four tokens: sixteen waves of one row
    // and two units per lane (13.41 / 14.62 / 14.99 against 14.12 / 17.58 /
    // 18.85 with seven units per lane)
    if (nu <= 2 && type == QMV_Q8_0 && n_tok == 4 && rpc <= 64)
      name = "fl_w8_r2_u2_l";
    else if (type == QMV_Q8_0 && nu >= 4 && nu <= 7 && n_tok >= 2 && rpc <= 16)
      name = "fl_w16_r1_u2_l";
    else if (nu <= 2)
      name = type == QMV_Q8_0 || type == QMV_Q8G128 ? "fl_w4_r1_u2_l"
             : type == QMV_Q4_K                      ? "fl_w4_r2_u2_l"
                                                     : "fl_w4_r2_u2_g";
    else
      name = nu <= 3 ? "fl_w16_r1_u3_l" : nu <= 7 ? "fl_w8_r1_u7_l" : "fl_w4_r1_u4_g";
  } else if (type == QMV_Q4_K && n_tok <= 8 && n_rows >= 8 * (int64_t)cus &&
             units * mx_per_unit(FQ4_K, 8) <= 140 * 1024) {
    // q4_K at 5..8 tokens on many rows (and 3, 4 on long rows): the flat
    // matrix-core kernel, one pass with every weight load of a wave issued
    // at once (14336 x 4096: 12.1 / 12.2 us at 5 / 8 tokens against 16.5 /
    // 17.8 for the flat vector kernel and 14.2 at 8 for the persistent
    // matrix-core kernel)
    name = "mf_w8_b4";
  } else if (type == QMV_Q4_K && n_tok == 3 && nu <= 2) {
    name = "fl_w4_r1_u2_l";  // measured 11.25 against 11.59 us for the multi-token kernel
  } else if (type == QMV_Q5_K || type == QMV_Q6_K) {
    // q5_K, q6_K (measured on 14336 x 4096 at 3..16 tokens): q6_K keeps the
    // flat kernel while one chunk covers the row, q5_K the multi-token one
    // from five tokens (us: q5_K at 3 / 4 two rows per wave 12.8 / 13.4
    // against 13.6 / 13.8 for the multi-token kernel; q6_K at 3 / 4 two rows
    // per wave 15.0 / 15.7 against 15.7 / 16.5 for one, at 6 / 8 / 12 / 16
    // eight waves of two rows 22.0 / 22.4 / 34.3 / 35.4 against 22.6 / 24.0 /
    // 35.9 / 37.4 for the other flat shapes, at 5 and 9 / 10 four waves of
    // two rows, 21.4 and 31.8 / 32.2 against 35.5 / 35.5 for sixteen of one)
    if (type == QMV_Q6_K && nu <= 2)
      name = n_tok <= 4                                       ? "fl_w4_r2_u2_l"
             : n_tok == 5 || (n_tok >= 9 && n_tok <= 10)      ? "fl_w4_r2_u2_g"
                                                              : "fl_w8_r2_u2_l";
    else if (type == QMV_Q5_K && nu <= 2 && n_tok <= 4)
      name = "fl_w4_r2_u2_l";
    else
      name = n_tok > 8 ? "mt_r4_w8_k2" : "mt_r2_w8_k2";
  } else if ((type == QMV_Q8_0 || type == QMV_Q8G128) && (n_tok <= 8 || rpc < 128)) {
    // Q8_0 at 5..8 tokens, Q8G128 at 3..8 (and both beyond on fewer than
    // 128 rows per compute unit, where the matrix-core kernel is slower):
    // measured on 152064x5120, 14336x4096, 4096x4096 and 4096x14336
    // (the heads, 152064 x 5120, at 5 / 6 / 7 / 8 tokens: the multi-token
    // kernel with two rows per lane group 175 / 180 / 184 / 188.5 us against
    // 191.5 / 194 / 195.5 / 198 for the flat one (Q8_0), 183 / 186.5 / 194 /
    // 196.5 against 193 / 194.5 / 196.7 / 198 (Q8G128); the flat one stays
    // ahead at 3 and 4 tokens: 149 against 153 us for Q8G128 at three)
    if (rpc >= 128)
      name = n_tok > 8    ? "mt_r4_w4_k1"
             : nu <= 2    ? "fl_w16_r1_u2_l"
             : n_tok >= 5 ? "mt_r2_w4_k1"
                          : "fl_w16_r1_u3_l";
    else if (rpc >= 32 && rpc < 48 && nu <= 2 && type == QMV_Q8_0)
      // 8192 x 4096: at 5 / 6 / 8 tokens eight waves of two rows 11.13 /
      // 11.06 / 12.35 us against 13.23 / 13.51 / 14.44 for the multi-token
      // kernel, at 10 / 16 the flat matrix-core kernel 15.38 / 15.36 against
      // 21.49 / 23.68
      name = n_tok <= 8 ? "fl_w8_r2_u2_l" : "mf_w8_b4";
    else if (rpc >= 32)
      name = "mt_r2_w4_k1";
    else if (nu <= 2 && n_tok <= 4)
      name = "fl_w4_r1_u2_l";
    else if (nu <= 2 && n_tok <= 7 && type == QMV_Q8_0)
      name = "fl_w8_r2_u2_l";  // 4096 x 4096 at 5 / 6 / 7 tokens: 7.46 / 7.54 / 7.69 us against 8.01 / 8.09 / 8.02
    else
      name = n_tok > 8 && nu > 2 ? "mt_r1_w8_k4" : "fl_w16_r1_u2_l";
  } else if (n_tok > 8) {
    const int64_t per = 16 * (int64_t)cus / tiles;  // waves of K split per row tile
    // (eight waves splitting K only from 16 waves of K split per row tile:
    // q4_K and IQ4_XS 8192 x 14336 at 10 / 16 tokens, unsplit, 29.4 / 30.2
    // and 28.0 / 28.3 us with four against 44.1 / 45.1 and 41.5 / 42.6 with
    // eight)
    name = per >= 16 ? "mx_w8_k8_r4" : per >= 4 ? "mx_w8_k4_r4" : "mx_w8_k1_r4";
  } else if (type == QMV_IQ4_XS || (type == QMV_Q4_K && n_tok > 4)) {
    // (8192 x 14336, 8 waves of K split per tile: q4_K at 5..8 tokens
    // sixteen-wave workgroups split four ways 21.7 against 22.6 us eight
    // ways; IQ4_XS at 3..8 eight-wave ones split four ways 18.6 at 3 and 4
    // tokens, 20.2 at 5, against 19.5 and 21.4 with sixteen split eight ways)
    const int64_t per = 16 * (int64_t)cus / tiles;
    name = per >= 16                        ? "mx_w16_k16_r2"
           : per >= 8 && type == QMV_IQ4_XS ? "mx_w8_k4_r4"
                                            : "mx_w16_k4_r2";
  } else {
    name = rpc >= 128 ? "mt_r4_w4_k1" : rpc >= 32 ? "mt_r2_w8_k2" : rpc >= 16 ? "mt_r2_w16_k8" : "mt_r1_w16_k8";
  }
  int v = find_variant(name);
  if (!stream_fits(v, k, n_tok)) v = find_variant("mt_r2_w8_k4");
  return v;
}

int choose_variant(int type, int64_t n_rows, int64_t k, int64_t n_tok) {
  const int64_t forced = g_variant.load();
  if (forced >= 0 && forced < kNumVariants && is_mx(kVariants[forced]) && !has_mfma(type))
    return auto_variant(type, n_rows, k, n_tok);  // no matrix-core decode of this format
  if (forced >= 0 && forced < kNumVariants) {
    // a forced streaming variant whose staging does not fit runs the
    // lane-group kernel instead
    return stream_fits((int)forced, k, n_tok) ? static_cast<int>(forced)
                                              : find_variant("lpr64_r2");
  }
  return auto_variant(type, n_rows, k, n_tok);
}

int choose_slices(const Variant& v, int64_t n_rows, int64_t k) {
  const int64_t units = k / 32;
  const int64_t forced = g_splitk.load();
  if (forced == 0) return 1;
  const int64_t max_by_units = units / v.lpr;  // >= one unit per lane per slice
  int64_t s;
  if (forced > 0) {
    s = forced;
  } else {
    const int64_t waves = (n_rows + (64 / v.lpr) * v.rows - 1) / ((64 / v.lpr) * v.rows);
    const int64_t want = 8 * static_cast<int64_t>(device_cus());  // ~8 waves per CU
    if (waves >= want / 2 || units < 4 * v.lpr) return 1;
    s = (want + waves - 1) / waves;
    s = s > units / (2 * v.lpr) ? units / (2 * v.lpr) : s;  // >= two units per lane
  }
  if (s > max_by_units) s = max_by_units;
  if (s > kMaxSlices) s = kMaxSlices;
  return s < 1 ? 1 : static_cast<int>(s);
}

// The kernel of a qmv_matvec call and its cross-workgroup K slices (1:
// none); split says whether the call uses the workspace.
struct Plan {
  int variant;
  int slices;
  bool split;
  int ups;  // flat kernel split: units per slice
};

// Flat-kernel (LDS-staged) split over workgroups: where the row is longer
// than one chunk (64 * nu units per lane) or the variant's workgroup columns
// leave compute units without a workgroup, slices of whole super-blocks of
// at most one chunk, as many as give every compute unit a workgroup.
// Returns the slice count (1: no split) and the units per slice in *ups.
int flat_split(const Variant& v, int64_t n_rows, int64_t units, int64_t n_tok, int* ups) {
  const int64_t ch = 64 * (int64_t)v.nu;
  const int64_t cols = (n_rows + (int64_t)v.wpb * v.rows - 1) / ((int64_t)v.wpb * v.rows);
  const int64_t cus = device_cus();
  const int64_t s_min = (units + ch - 1) / ch;
  const int64_t fill = (cus + cols - 1) / cols;
  int64_t s = s_min > fill ? s_min : fill;
  if (s < 2) return 1;
  int64_t u = ((units + s - 1) / s + 7) / 8 * 8;
  if (u > ch) u = ch / 8 * 8;
  s = (units + u - 1) / u;
  if (s < 2 || s > kMaxSlices || n_tok * u * 40 > device_info().lds_per_block) return 1;
  *ups = static_cast<int>(u);
  return static_cast<int>(s);
}

// With a workspace, rows too long for one LDS chunk on few row tiles run the
// matrix-core variant measured fastest split over workgroups (4096 x 14336:
// IQ4_XS 16 tokens 25.3 -> 19.4 us; q4_K at 10 / 16 tokens 22.8 / 25.2 us
// with eight-wave workgroups, 16.9 / 17.3 with sixteen since the two-phase
// step fits them in 128 VGPRs; q4_K 8 tokens 18.5 -> 16.1 us), when its plan
// splits; -1 otherwise.
// At 9-16 tokens the sixteen-wave kernel splits only on few row tiles; on
// more (8192 x 14336) the eight-wave one with one wave per tile split four
// ways is next (26.2 / 27.9 us at 10 / 16 tokens against 29.4 / 30.2
// unsplit).
int split_variant(int type, int64_t n_rows, int64_t k, int64_t n_tok) {
  const bool k4iq = type == QMV_IQ4_XS || type == QMV_Q4_K;
  const char* names[2] = {n_tok > 8 && k4iq ? "mx_w16_k4_r2" : type == QMV_Q4_K && n_tok > 4 ? "mx_w8_k4_r4" : nullptr,
                          n_tok > 8 && k4iq ? "mx_w8_k1_r4" : nullptr};
  const DeviceInfo dv = device_info();
  for (const char* name : names) {
    if (name == nullptr) continue;
    const int v = find_variant(name);
    int ups = 0;
    if (mx_split_plan(type, (int)n_tok, kVariants[v].wpb, kVariants[v].ks, (int)(k / 32), (int)n_rows, dv.cus,
                      dv.lds_per_cu, mx_slices(), &ups) >= 2)
      return v;
  }
  return -1;
}

Plan make_plan(int type, int64_t n_rows, int64_t k, int64_t n_tok, bool use_ws) {
  Plan p{choose_variant(type, n_rows, k, n_tok), 1, false, 0};
  if (!use_ws || g_splitk.load() == 0) return p;
  p.split = true;
  // forced slices belong to the lane-group kernel's split (the streaming
  // kernels split K inside a workgroup and need no workspace)
  if (g_splitk.load() > 0 && kVariants[p.variant].kind != 0) p.variant = find_variant("lpr64_r2");
  if (kVariants[p.variant].kind == 0) {
    p.slices = choose_slices(kVariants[p.variant], n_rows, k);
  } else if (kVariants[p.variant].kind == 4) {
    if (g_variant.load() < 0) {
      const int sv = split_variant(type, n_rows, k, n_tok);
      if (sv >= 0) p.variant = sv;
    }
    const DeviceInfo dv = device_info();
    int ups = 0;
    const int s = mx_split_plan(type, (int)n_tok, kVariants[p.variant].wpb, kVariants[p.variant].ks, (int)(k / 32),
                                (int)n_rows, dv.cus, dv.lds_per_cu, mx_slices(), &ups);
    p.slices = s >= 2 ? s : 1;
  } else if (kVariants[p.variant].kind == 5) {
    // the flat matrix-core kernel's own plan (launch_matvec repeats it)
    const DeviceInfo dv = device_info();
    MxfPlan mp{};
    const int s = mxf_plan(type, (int)n_tok, kVariants[p.variant].wpb, kVariants[p.variant].nu, (int)(k / 32),
                           (int)n_rows, dv.cus, dv.lds_per_cu, mx_slices() != 0, mx_slices() >= 2 ? mx_slices() : 0,
                           &mp);
    p.slices = s >= 1 ? s : 1;
  } else if (kVariants[p.variant].kind == 2 && kVariants[p.variant].xl && flat_split_enabled()) {
    p.slices = flat_split(kVariants[p.variant], n_rows, k / 32, n_tok, &p.ups);
  }
  return p;
}

// Split-K workspace: [one counter per row tile][partials slices x T x N].
// The counter area has a fixed size (every variant covers >= 4 rows per
// workgroup, and split-K is limited to kSplitMaxRows rows), so calls of
// different shapes can share one workspace: a call's partials never land on
// the counters of another.
constexpr int64_t kSplitCounterBytes = kSplitMaxRows;  // kSplitMaxRows / 4 ints

// MoE workspace: [256 B status][reserved area][per-slot outputs of the
// route-weighted combine], at fixed offsets so that calls of different shapes
// can share one workspace.
constexpr int64_t kMoeMaxRows = 65536;
constexpr int64_t kMoeStatusBytes = 256;
constexpr int64_t kMoeCounterBytes = kMoeMaxRows;  // kMoeMaxRows / 4 ints
constexpr int64_t kMoePartOffset = kMoeStatusBytes + kMoeCounterBytes;

}  // namespace

// The last HIP error an entry point of this thread turned into QMV_ERR_HIP.
static thread_local hipError_t g_last_hip = hipSuccess;

static qmv_status hip_status(hipError_t e) {
  if (e == hipSuccess) return QMV_OK;
  g_last_hip = e;
  return QMV_ERR_HIP;
}

// ------------------------------------------------------------------ misc
QMV_API int qmv_abi_version(void) { return QMV_ABI_VERSION; }

QMV_API int qmv_last_hip_error(void) { return static_cast<int>(g_last_hip); }

QMV_API const char* qmv_last_hip_error_name(void) {
  return g_last_hip == hipSuccess ? "hipSuccess" : hipGetErrorName(g_last_hip);
}

QMV_API const char* qmv_status_string(qmv_status st) {
  switch (st) {
    case QMV_OK: return "QMV_OK";
    case QMV_ERR_INVALID_ARG: return "QMV_ERR_INVALID_ARG: invalid argument";
    case QMV_ERR_UNSUPPORTED: return "QMV_ERR_UNSUPPORTED: outside the supported range";
    case QMV_ERR_MISALIGNED: return "QMV_ERR_MISALIGNED: pointer alignment";
    case QMV_ERR_WORKSPACE: return "QMV_ERR_WORKSPACE: workspace missing or too small";
    case QMV_ERR_HIP: return "QMV_ERR_HIP: HIP runtime error";
    default: return "unknown qmv status";
  }
}

QMV_API size_t qmv_row_bytes(qmv_type type, int64_t k) {
  if (!valid_type(type) || k < 1 || k % block_k(type)) return 0;
  return static_cast<size_t>(k / block_k(type) * block_bytes(type));
}

QMV_API size_t qmv_act_offset_d(int64_t n_tok, int64_t k) {
  if (n_tok < 1 || k < 1 || k % 32) return 0;
  return static_cast<size_t>(align256(n_tok * k));
}
QMV_API size_t qmv_act_offset_s(int64_t n_tok, int64_t k) {
  if (n_tok < 1 || k < 1 || k % 32) return 0;
  return static_cast<size_t>(align256(n_tok * k) + align256(n_tok * (k / 32) * 4));
}
QMV_API size_t qmv_act_bytes(int64_t n_tok, int64_t k) {
  if (n_tok < 1 || k < 1 || k % 32) return 0;
  return static_cast<size_t>(align256(n_tok * k) + 2 * align256(n_tok * (k / 32) * 4));
}

QMV_API qmv_status qmv_set_tuning(const char* key, int64_t value) {
  if (key == nullptr) return QMV_ERR_INVALID_ARG;
  if (!std::strcmp(key, "splitk")) {
    if (value < -1) return QMV_ERR_INVALID_ARG;
    g_splitk = value;
    return QMV_OK;
  }
  if (!std::strcmp(key, "mx_slices")) {
    if (value < -1 || value == 1 || value > kMaxSlices) return QMV_ERR_INVALID_ARG;
    set_mx_slices(static_cast<int>(value));
    return QMV_OK;
  }
  if (!std::strcmp(key, "flat_split")) {
    if (value < 0 || value > 1) return QMV_ERR_INVALID_ARG;
    g_flat_split = value;
    return QMV_OK;
  }
  if (!std::strcmp(key, "bpc")) {
    if (value < 0 || value > 64) return QMV_ERR_INVALID_ARG;
    set_blocks_per_cu(static_cast<int>(value));
    return QMV_OK;
  }
  if (!std::strcmp(key, "moe_kernel")) {
    if (value < 0 || value > 3) return QMV_ERR_INVALID_ARG;
    set_moe_kernel(static_cast<int>(value));
    return QMV_OK;
  }
  if (!std::strcmp(key, "moe_row16")) {
    if (value < 0 || value > 1) return QMV_ERR_INVALID_ARG;
    set_moe_row16(static_cast<int>(value));
    return QMV_OK;
  }
  if (!std::strcmp(key, "ffn_fuse")) {
    if (value < -1 || value > 1) return QMV_ERR_INVALID_ARG;
    g_ffn_fuse = value;
    return QMV_OK;
  }
  if (!std::strcmp(key, "variant")) {
    if (value < -1 || value >= kNumVariants) return QMV_ERR_INVALID_ARG;
    g_variant = value;
    return QMV_OK;
  }
  return QMV_ERR_INVALID_ARG;
}

QMV_API const char* qmv_variant_name(int64_t index) {
  return (index >= 0 && index < kNumVariants) ? kVariants[index].name : nullptr;
}

QMV_API int64_t qmv_pick_variant(qmv_type type, int64_t n_rows, int64_t k, int64_t n_tok) {
  if (!valid_type(type) || n_rows < 1 || k < 1 || k % block_k(type) || n_tok < 1 ||
      n_tok > QMV_MAX_TOKENS)
    return -1;
  return choose_variant(type, n_rows, k, n_tok);
}

QMV_API qmv_status qmv_matvec_plan(qmv_type type, int64_t n_rows, int64_t k, int64_t n_tok, int with_workspace,
                                   int64_t* variant, int* slices) {
  if (!valid_type(type) || n_rows < 1 || k < 1 || k % block_k(type) || n_tok < 1 || variant == nullptr ||
      slices == nullptr)
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_TOKENS) return QMV_ERR_UNSUPPORTED;
  const bool use_ws = with_workspace != 0 && qmv_matvec_workspace_bytes(type, n_rows, k, n_tok) > 0;
  const Plan p = make_plan(type, n_rows, k, n_tok, use_ws);
  *variant = p.variant;
  *slices = p.slices;
  return QMV_OK;
}

// ------------------------------------------------------------- quantize
QMV_API qmv_status qmv_quantize_act(const float* x, int64_t ldx, int64_t n_tok, int64_t k,
                                    void* xq, void* stream) {
  if (x == nullptr || xq == nullptr || n_tok < 1 || k < 1 || k % 32 || ldx < k)
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_ACT_ROWS || k > (int64_t)1 << 24) return QMV_ERR_UNSUPPORTED;
  // each lane reads four values with one 16-byte load at x + t * ldx + 4j
  if (!aligned(x, 16) || ldx % 4 || !aligned(xq, 256)) return QMV_ERR_MISALIGNED;
  uint8_t* b = static_cast<uint8_t*>(xq);
  hipError_t e = launch_quantize(x, ldx, static_cast<int>(n_tok), static_cast<int>(k),
                                 reinterpret_cast<int8_t*>(b),
                                 reinterpret_cast<float*>(b + qmv_act_offset_d(n_tok, k)),
                                 reinterpret_cast<int32_t*>(b + qmv_act_offset_s(n_tok, k)),
                                 static_cast<hipStream_t>(stream));
  return hip_status(e);
}

QMV_API qmv_status qmv_swiglu_quantize(const float* gu, int64_t ldg, int64_t rows, int64_t n_ff,
                                       void* xq, float* h_out, void* stream) {
  if (gu == nullptr || xq == nullptr || rows < 1 || n_ff < 1 || n_ff % 32 || ldg < 2 * n_ff)
    return QMV_ERR_INVALID_ARG;
  if (rows > QMV_MAX_ACT_ROWS || n_ff > (int64_t)1 << 24) return QMV_ERR_UNSUPPORTED;
  // each lane reads four values of g and of u with 16-byte loads
  if (!aligned(gu, 16) || ldg % 4 || !aligned(xq, 256) || (h_out != nullptr && !aligned(h_out, 16)))
    return QMV_ERR_MISALIGNED;
  uint8_t* b = static_cast<uint8_t*>(xq);
  hipError_t e = launch_swiglu_quantize(gu, ldg, static_cast<int>(rows), static_cast<int>(n_ff),
                                        reinterpret_cast<int8_t*>(b),
                                        reinterpret_cast<float*>(b + qmv_act_offset_d(rows, n_ff)),
                                        reinterpret_cast<int32_t*>(b + qmv_act_offset_s(rows, n_ff)), h_out,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e);
}

QMV_API qmv_status qmv_router_topk(const float* x, int64_t ldx, int64_t n_tok, int64_t k, const float* wr,
                                   int64_t n_experts, int64_t top_k, int32_t* ids, float* weights,
                                   float* logits, void* xq, void* stream) {
  if (x == nullptr || wr == nullptr || ids == nullptr || weights == nullptr || logits == nullptr || n_tok < 1 ||
      k < 1 ||
      k % 4 || ldx < k || ldx % 4 || n_experts < 1 || top_k < 1 || top_k > n_experts || (xq != nullptr && k % 32))
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_MOE_TOKENS || k > (int64_t(1) << 24) || n_experts > QMV_MAX_EXPERTS ||
      top_k > QMV_MAX_TOP_K)
    return QMV_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(wr, 16) || !aligned(ids, 4) || !aligned(weights, 4) || !aligned(logits, 4) ||
      (xq != nullptr && !aligned(xq, 256)))
    return QMV_ERR_MISALIGNED;
  ActView xv{};
  if (xq != nullptr) xv = act_view(xq, n_tok, k);
  hipError_t e = launch_router_topk(x, ldx, static_cast<int>(n_tok), static_cast<int>(k), wr,
                                    static_cast<int>(n_experts), static_cast<int>(top_k), ids, weights, logits,
                                    const_cast<int8_t*>(xv.qs), const_cast<float*>(xv.d),
                                    const_cast<int32_t*>(xv.s), static_cast<hipStream_t>(stream));
  return hip_status(e);
}

// --------------------------------------------------------------- matvec
QMV_API size_t qmv_matvec_workspace_bytes(qmv_type type, int64_t n_rows, int64_t k,
                                          int64_t n_tok) {
  if (!valid_type(type) || n_rows < 1 || k < 1 || k % block_k(type) || n_tok < 1 ||
      n_tok > QMV_MAX_TOKENS)
    return 0;
  if (n_rows > kSplitMaxRows) return 0;  // never split: no workspace needed
  return static_cast<size_t>(kSplitCounterBytes +
                             align256(int64_t(kMaxSlices) * n_tok * n_rows * 4));
}

QMV_API qmv_status qmv_matvec(qmv_type type, const void* w, int64_t n_rows, int64_t k,
                              const void* xq, int64_t n_tok, float* y, int64_t ldy, void* ws,
                              size_t ws_bytes, void* stream) {
  qmv_status st = check_weights(type, w, n_rows, k);
  if (st != QMV_OK) return st;
  if (xq == nullptr || y == nullptr || ldy < n_rows || n_tok < 1) return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_TOKENS) return QMV_ERR_UNSUPPORTED;
  if (!aligned(xq, 256) || !aligned(y, 4)) return QMV_ERR_MISALIGNED;
  MatvecLaunch a{};
  a.fmt = type;
  a.w = static_cast<const uint8_t*>(w);
  a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
  a.n_rows = static_cast<int>(n_rows);
  a.units = static_cast<int>(k / 32);
  a.x = act_view(xq, n_tok, k);
  a.n_tok = static_cast<int>(n_tok);
  a.y = y;
  a.ldy = ldy;
  a.xq = static_cast<const uint8_t*>(xq);
  a.act_bytes = static_cast<int64_t>(qmv_act_bytes(n_tok, k));
  a.off_d = static_cast<int64_t>(qmv_act_offset_d(n_tok, k));
  a.off_s = static_cast<int64_t>(qmv_act_offset_s(n_tok, k));
  const DeviceInfo dv = device_info();
  a.cus = dv.cus;
  a.lds_per_cu = dv.lds_per_cu;
  const size_t need = qmv_matvec_workspace_bytes(type, n_rows, k, n_tok);
  const bool use_ws = ws != nullptr && need > 0;
  if (use_ws) {
    if (ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return QMV_ERR_MISALIGNED;
  }
  const Plan p = make_plan(type, n_rows, k, n_tok, use_ws);
  a.variant = p.variant;
  a.slices = kVariants[p.variant].kind == 0 ? p.slices : 1;  // k_mx plans its own split
  if (kVariants[p.variant].kind == 2 && p.slices > 1) {
    a.fslices = p.slices;
    a.fups = p.ups;
  }
  if (p.split) {
    uint8_t* b = static_cast<uint8_t*>(ws);
    a.cnt = reinterpret_cast<int*>(b);
    a.part = reinterpret_cast<float*>(b + kSplitCounterBytes);
  }
  hipError_t e = launch_matvec(a, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

// The LDS-staged flat variant that quantizes its own activations for a
// shape, or -1 for two launches.  Every workgroup re-reads and re-quantizes
// all of x before its weights can be used, which only pays for short rows
// and few tokens: measured on MI355X, Q8_0 4096 x 4096 at 1 / 2 tokens went
// 7.4 -> 5.6 / 8.0 -> 6.6 us per step and q4_K 14336 x 4096 at one token
// 10.0 -> 9.8 us, while q4_K at two tokens and IQ4_XS 4096 x 14336 were
// slower fused.  So: sixteen-wave workgroups (the fewest quantizing copies),
// Q8_0 at up to two tokens and q4_K at one, rows of at most 128 blocks.  A
// forced LDS-staged flat variant is honoured (tests).
static int fused_variant(int type, int64_t n_rows, int64_t k, int64_t n_tok) {
  if (n_tok > 2) return -1;
  const int64_t forced = g_variant.load();
  int v = -1;
  if (forced >= 0 && forced < kNumVariants && kVariants[forced].kind == 2 && kVariants[forced].xl)
    v = static_cast<int>(forced);
  else if (k / 32 <= 128 && n_rows >= 4 * (int64_t)device_cus() && type == QMV_Q8_0)
    v = find_variant("fl_w16_r1_u2_l");
  else if (k / 32 <= 128 && n_rows >= 4 * (int64_t)device_cus() && type == QMV_Q4_K && n_tok == 1)
    v = find_variant("fl_w16_r2_u2_l");
  if (v < 0 || !stream_fits(v, k, n_tok)) return -1;
  return v;
}

QMV_API qmv_status qmv_matvec_x(qmv_type type, const void* w, int64_t n_rows, int64_t k, const float* x,
                                int64_t ldx, int64_t n_tok, float* y, int64_t ldy, void* xq, void* ws,
                                size_t ws_bytes, void* stream) {
  qmv_status st = check_weights(type, w, n_rows, k);
  if (st != QMV_OK) return st;
  if (x == nullptr || xq == nullptr || y == nullptr || ldy < n_rows || n_tok < 1 || ldx < k || ldx % 4)
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_TOKENS) return QMV_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(xq, 256) || !aligned(y, 4)) return QMV_ERR_MISALIGNED;
  // the workspace as qmv_matvec checks it, before the quantizer is enqueued
  const size_t need = qmv_matvec_workspace_bytes(type, n_rows, k, n_tok);
  if (ws != nullptr && need > 0) {
    if (ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return QMV_ERR_MISALIGNED;
  }
  const int v = fused_variant(type, n_rows, k, n_tok);
  if (v < 0) {  // two launches
    st = qmv_quantize_act(x, ldx, n_tok, k, xq, stream);
    if (st != QMV_OK) return st;
    return qmv_matvec(type, w, n_rows, k, xq, n_tok, y, ldy, ws, ws_bytes, stream);
  }
  MatvecLaunch a{};
  a.fmt = type;
  a.w = static_cast<const uint8_t*>(w);
  a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
  a.n_rows = static_cast<int>(n_rows);
  a.units = static_cast<int>(k / 32);
  a.x = act_view(xq, n_tok, k);
  a.n_tok = static_cast<int>(n_tok);
  a.y = y;
  a.ldy = ldy;
  a.qx = true;
  a.xf = x;
  a.ldx = ldx;
  a.variant = v;
  a.slices = 1;
  a.xq = static_cast<const uint8_t*>(xq);
  a.act_bytes = static_cast<int64_t>(qmv_act_bytes(n_tok, k));
  a.off_d = static_cast<int64_t>(qmv_act_offset_d(n_tok, k));
  a.off_s = static_cast<int64_t>(qmv_act_offset_s(n_tok, k));
  const DeviceInfo dv = device_info();
  a.cus = dv.cus;
  a.lds_per_cu = dv.lds_per_cu;
  hipError_t e = launch_matvec(a, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

// Byte extent [lo, hi) of an fp32 [n_tok][ld] output touching n columns.
static void extent(const float* p, int64_t n_tok, int64_t ld, int64_t n, uintptr_t& lo, uintptr_t& hi) {
  lo = reinterpret_cast<uintptr_t>(p);
  hi = lo + static_cast<uintptr_t>(((n_tok - 1) * ld + n) * 4);
}

QMV_API qmv_status qmv_matvec_batch(qmv_type type, const qmv_matvec_item* items, int64_t n_items,
                                    int64_t k, const void* xq, int64_t n_tok, void* stream) {
  if (!valid_type(type) || items == nullptr || n_items < 1 || xq == nullptr || n_tok < 1)
    return QMV_ERR_INVALID_ARG;
  if (n_items > QMV_MAX_BATCH || n_tok > QMV_MAX_TOKENS) return QMV_ERR_UNSUPPORTED;
  static_assert(QMV_MAX_BATCH <= kMaxBatch, "segment table");
  MatvecLaunch a{};
  int64_t rows = 0;  // launch rows so far (each matrix starts on a kSegAlign boundary)
  for (int64_t i = 0; i < n_items; ++i) {
    const qmv_matvec_item& it = items[i];
    const qmv_status st = check_weights(type, it.w, it.n_rows, k);
    if (st != QMV_OK) return st;
    if (it.y == nullptr || it.ldy < it.n_rows || (it.residual != nullptr && it.ldr < it.n_rows))
      return QMV_ERR_INVALID_ARG;
    if (!aligned(it.y, 4) || (it.residual != nullptr && !aligned(it.residual, 4))) return QMV_ERR_MISALIGNED;
    rows = (rows + kSegAlign - 1) / kSegAlign * kSegAlign;
    RowSeg& sg = a.seg.s[i];
    sg.first = static_cast<int>(rows);
    sg.rows = static_cast<int>(it.n_rows);
    sg.w = static_cast<const uint8_t*>(it.w);
    sg.y = it.y;
    sg.ldy = it.ldy;
    sg.res = it.residual;
    sg.ldr = it.residual != nullptr ? it.ldr : 0;
    rows += it.n_rows;
    if (rows > INT32_MAX / 4) return QMV_ERR_INVALID_ARG;
  }
  // outputs pairwise disjoint; a residual is its own output or disjoint from all
  for (int64_t i = 0; i < n_items; ++i) {
    uintptr_t lo, hi;
    extent(items[i].y, n_tok, items[i].ldy, items[i].n_rows, lo, hi);
    for (int64_t j = 0; j < n_items; ++j) {
      uintptr_t l2, h2;
      if (j != i) {
        extent(items[j].y, n_tok, items[j].ldy, items[j].n_rows, l2, h2);
        if (lo < h2 && l2 < hi) return QMV_ERR_INVALID_ARG;
      }
      const float* r = items[j].residual;
      if (r == nullptr || (j == i && r == items[i].y && items[i].ldr == items[i].ldy)) continue;
      extent(r, n_tok, items[j].ldr, items[j].n_rows, l2, h2);
      if (lo < h2 && l2 < hi) return QMV_ERR_INVALID_ARG;
    }
  }
  if (!aligned(xq, 256)) return QMV_ERR_MISALIGNED;
  a.seg.n = static_cast<int>(n_items);
  a.fmt = type;
  a.w = a.seg.s[0].w;
  a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
  a.n_rows = static_cast<int>(rows);
  a.units = static_cast<int>(k / 32);
  a.x = act_view(xq, n_tok, k);
  a.n_tok = static_cast<int>(n_tok);
  a.y = a.seg.s[0].y;
  a.ldy = a.seg.s[0].ldy;
  // the lane-group kernel (kind 0) has no segment table: a forced variant of
  // that kind gives way to the automatic choice
  a.variant = choose_variant(type, rows, k, n_tok);
  if (kVariants[a.variant].kind == 0) a.variant = auto_variant(type, rows, k, n_tok);
  a.slices = 1;
  a.xq = static_cast<const uint8_t*>(xq);
  a.act_bytes = static_cast<int64_t>(qmv_act_bytes(n_tok, k));
  a.off_d = static_cast<int64_t>(qmv_act_offset_d(n_tok, k));
  a.off_s = static_cast<int64_t>(qmv_act_offset_s(n_tok, k));
  const DeviceInfo dv = device_info();
  a.cus = dv.cus;
  a.lds_per_cu = dv.lds_per_cu;
  hipError_t e = launch_matvec(a, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

QMV_API qmv_status qmv_block_dots(qmv_type type, const void* w, int64_t n_rows, int64_t k,
                                  const void* xq, int64_t n_tok, int32_t* out, void* stream) {
  qmv_status st = check_weights(type, w, n_rows, k);
  if (st != QMV_OK) return st;
  if (xq == nullptr || out == nullptr || n_tok < 1) return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_TOKENS) return QMV_ERR_UNSUPPORTED;
  if (n_tok * n_rows * (k / 32) > INT32_MAX) return QMV_ERR_UNSUPPORTED;
  if (!aligned(xq, 256) || !aligned(out, 4)) return QMV_ERR_MISALIGNED;
  hipError_t e = launch_block_dots(type, static_cast<const uint8_t*>(w),
                                   static_cast<int64_t>(qmv_row_bytes(type, k)),
                                   static_cast<int>(n_rows), static_cast<int>(k / 32),
                                   act_view(xq, n_tok, k), static_cast<int>(n_tok), out,
                                   static_cast<hipStream_t>(stream));
  return hip_status(e);
}

QMV_API qmv_status qmv_block_dots_mx(qmv_type type, const void* w, int64_t n_rows, int64_t k, const void* xq,
                                     int64_t n_tok, int64_t variant, int slices, int32_t* out, void* stream) {
  qmv_status st = check_weights(type, w, n_rows, k);
  if (st != QMV_OK) return st;
  if (xq == nullptr || out == nullptr || n_tok < 1 || slices < -1 || slices == 1 || slices > kMaxSlices ||
      variant < -1 || variant >= kNumVariants || (variant >= 0 && !is_mx(kVariants[variant])))
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_TOKENS || !has_mfma(type)) return QMV_ERR_UNSUPPORTED;
  if (n_tok * n_rows * (k / 32) > INT32_MAX) return QMV_ERR_UNSUPPORTED;
  if (!aligned(xq, 256) || !aligned(out, 4)) return QMV_ERR_MISALIGNED;
  int v = static_cast<int>(variant);
  if (v < 0) {
    // the matrix-core variant qmv_matvec runs for this shape with a
    // workspace, if it runs one; else the 16-wave one up to eight tokens
    // and the 8-wave one beyond
    const bool use_ws = qmv_matvec_workspace_bytes(type, n_rows, k, n_tok) > 0;
    const Plan p = make_plan(type, n_rows, k, n_tok, use_ws);
    v = is_mx(kVariants[p.variant]) ? p.variant : find_variant(n_tok <= 8 ? "mx_w16_k4_r2" : "mx_w8_k1_r4");
  }
  const DeviceInfo dv = device_info();
  MxfPlan mp{};
  if (kVariants[v].kind == 5) {
    // the flat matrix-core kernel: its plan with that many slices (-1 the
    // automatic one, 0 unsplit)
    if (mxf_plan(type, (int)n_tok, kVariants[v].wpb, kVariants[v].nu, (int)(k / 32), (int)n_rows, dv.cus,
                 dv.lds_per_cu, slices != 0, slices >= 2 ? slices : 0, &mp) < 1)
      return QMV_ERR_UNSUPPORTED;
  } else if (slices >= 2) {
    int ups = 0;
    if (mx_split_plan(type, (int)n_tok, kVariants[v].wpb, kVariants[v].ks, (int)(k / 32), (int)n_rows, dv.cus,
                      dv.lds_per_cu, slices, &ups) < 2)
      return QMV_ERR_UNSUPPORTED;  // that many slices do not fit this shape
  }
  MatvecLaunch a{};
  a.fmt = type;
  a.w = static_cast<const uint8_t*>(w);
  a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
  a.n_rows = static_cast<int>(n_rows);
  a.units = static_cast<int>(k / 32);
  a.x = act_view(xq, n_tok, k);
  a.n_tok = static_cast<int>(n_tok);
  a.y = nullptr;
  a.ldy = n_rows;
  a.xq = static_cast<const uint8_t*>(xq);
  a.act_bytes = static_cast<int64_t>(qmv_act_bytes(n_tok, k));
  a.off_d = static_cast<int64_t>(qmv_act_offset_d(n_tok, k));
  a.off_s = static_cast<int64_t>(qmv_act_offset_s(n_tok, k));
  a.cus = dv.cus;
  a.lds_per_cu = dv.lds_per_cu;
  a.variant = v;
  a.slices = 1;
  a.dots = out;
  a.dots_slices = slices;
  hipError_t e = kVariants[v].kind == 5 ? launch_mxf(a, mp, static_cast<hipStream_t>(stream))
                                        : launch_mx(a, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

QMV_API qmv_status qmv_stream_read(const void* p, int64_t bytes, uint32_t* sink, void* stream) {
  if (p == nullptr || sink == nullptr || bytes < 16 || bytes % 16) return QMV_ERR_INVALID_ARG;
  if (bytes / 16 > (int64_t)INT32_MAX * 1024) return QMV_ERR_UNSUPPORTED;  // grid limit
  if (!aligned(p, 16) || !aligned(sink, 4)) return QMV_ERR_MISALIGNED;
  hipError_t e = launch_stream_read(static_cast<const uint8_t*>(p), bytes, 0x9e3779b9u, sink,
                                    static_cast<hipStream_t>(stream));
  return hip_status(e);
}

// ------------------------------------------------------------------ MoE
QMV_API size_t qmv_moe_workspace_bytes(qmv_type type, int64_t n_experts, int64_t n_rows,
                                       int64_t k, int64_t n_tok, int64_t top_k) {
  if (!valid_type(type) || !moe_format(type) || n_rows < 1 || k < 1 || k % block_k(type) || n_tok < 1 ||
      n_tok > QMV_MAX_MOE_TOKENS || top_k < 1 || top_k > QMV_MAX_TOP_K || n_experts < 1 ||
      n_experts > QMV_MAX_EXPERTS || k / 32 > kMoeMaxUnits || n_rows > kMoeMaxRows)
    return 0;
  return static_cast<size_t>(kMoePartOffset + align256(n_tok * top_k * n_rows * 4));
}

// Validation of a qmv_moe_matvec call, the workspace aside.
static qmv_status moe_check(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows, int64_t k,
                            const void* xq, int x_per_slot, const int32_t* ids, const float* route_w,
                            int64_t n_tok, int64_t top_k, float* y) {
  qmv_status st = check_weights(type, w, n_rows, k);
  if (st != QMV_OK) return st;
  if (xq == nullptr || ids == nullptr || y == nullptr || n_tok < 1 || top_k < 1 || n_experts < 1 ||
      (x_per_slot != 0 && x_per_slot != 1))
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_MOE_TOKENS || top_k > QMV_MAX_TOP_K || n_experts > QMV_MAX_EXPERTS ||
      k / 32 > kMoeMaxUnits || n_rows > kMoeMaxRows || !moe_format(type))
    return QMV_ERR_UNSUPPORTED;
  if (n_experts * n_rows > INT32_MAX) return QMV_ERR_UNSUPPORTED;
  if (!aligned(xq, 256) || !aligned(ids, 4) || !aligned(y, 4) || (route_w != nullptr && !aligned(route_w, 4)))
    return QMV_ERR_MISALIGNED;
  return QMV_OK;
}

// The launch of a validated qmv_moe_matvec call on workspace ws.
static qmv_status moe_run(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows, int64_t k,
                          const void* xq, int x_per_slot, const int32_t* ids, const float* route_w, int64_t n_tok,
                          int64_t top_k, float* y, void* ws, void* stream) {
  const int64_t x_rows = x_per_slot ? n_tok * top_k : n_tok;
  MoeLaunch a{};
  a.fmt = type;
  a.w = static_cast<const uint8_t*>(w);
  a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
  a.n_experts = static_cast<int>(n_experts);
  a.n_rows = static_cast<int>(n_rows);
  a.units = static_cast<int>(k / 32);
  a.x = act_view(xq, x_rows, k);
  a.x_rows = static_cast<int>(x_rows);
  a.x_per_slot = x_per_slot;
  a.ids = ids;
  a.rw = route_w;
  a.n_tok = static_cast<int>(n_tok);
  a.top_k = static_cast<int>(top_k);
  a.y = y;
  const DeviceInfo dv = device_info();
  a.cus = dv.cus;
  a.lds_per_cu = dv.lds_per_cu;
  uint8_t* b = static_cast<uint8_t*>(ws);
  a.err = reinterpret_cast<int*>(b);
  a.part = reinterpret_cast<float*>(b + kMoePartOffset);
  hipError_t e = launch_moe(a, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

QMV_API qmv_status qmv_moe_matvec(qmv_type type, const void* w, int64_t n_experts,
                                  int64_t n_rows, int64_t k, const void* xq, int x_per_slot,
                                  const int32_t* ids, const float* route_w, int64_t n_tok,
                                  int64_t top_k, float* y, void* ws, size_t ws_bytes,
                                  void* stream) {
  qmv_status st = moe_check(type, w, n_experts, n_rows, k, xq, x_per_slot, ids, route_w, n_tok, top_k, y);
  if (st != QMV_OK) return st;
  if (ws == nullptr) return QMV_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return QMV_ERR_MISALIGNED;
  if (ws_bytes < qmv_moe_workspace_bytes(type, n_experts, n_rows, k, n_tok, top_k)) return QMV_ERR_WORKSPACE;
  return moe_run(type, w, n_experts, n_rows, k, xq, x_per_slot, ids, route_w, n_tok, top_k, y, ws, stream);
}

QMV_API qmv_status qmv_moe_gate_up_swiglu(qmv_type type, const void* w, int64_t n_experts, int64_t n_ff, int64_t k,
                                          const void* xq, const int32_t* ids, int64_t n_tok, int64_t top_k, void* hq,
                                          float* gu, void* ws, size_t ws_bytes, void* stream) {
  if (hq == nullptr || n_ff < 1 || n_ff % 32 || n_ff > kMoeMaxRows / 2) return QMV_ERR_INVALID_ARG;
  // the routed gate+up call this stands for, validated as qmv_moe_matvec validates it
  float* y_check = gu != nullptr ? gu : reinterpret_cast<float*>(hq);
  qmv_status st = moe_check(type, w, n_experts, 2 * n_ff, k, xq, 0, ids, nullptr, n_tok, top_k, y_check);
  if (st != QMV_OK) return st;
  if (ws == nullptr) return QMV_ERR_INVALID_ARG;
  if (!aligned(ws, 256) || !aligned(hq, 256) || (gu != nullptr && !aligned(gu, 16))) return QMV_ERR_MISALIGNED;
  if (ws_bytes < qmv_moe_workspace_bytes(type, n_experts, 2 * n_ff, k, n_tok, top_k)) return QMV_ERR_WORKSPACE;
  const int64_t rows = n_tok * top_k;
  uint8_t* b = static_cast<uint8_t*>(ws);
  // One launch only when asked for: measured on the 128-expert IQ4_XS FFN
  // (3072 x 4096 gate+up, 4096 x 1536 down, top-8), the whole step took
  // 36.5 / 127.2 / 261.7 us at 1 / 6 / 16 tokens with it against
  // 34.8 / 119.6 / 235.5 us with two launches: its 1024-thread workgroups
  // (one per compute unit at its register count) and the barrier per slot
  // cost more than the second launch.  (Counting a block's 16 waves on a
  // device-scope arrival counter instead, in the 256-thread kernel, was
  // slower still: 52.2 / 129.8 / 261.5 us.)
  // (only where the routed matvec runs the few-slot kernel, whose sums the
  // one-launch kernel reproduces bit for bit)
  const bool fused = g_ffn_fuse.load() == 1 && k / 32 <= 128 && n_tok <= 16 &&
                     (moe_kernel() == 0 || moe_kernel() == 3);
  if (fused) {
    MoeLaunch a{};
    a.fmt = type;
    a.w = static_cast<const uint8_t*>(w);
    a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
    a.n_experts = static_cast<int>(n_experts);
    a.n_rows = static_cast<int>(2 * n_ff);
    a.units = static_cast<int>(k / 32);
    a.x = act_view(xq, n_tok, k);
    a.x_rows = static_cast<int>(n_tok);
    a.x_per_slot = 0;
    a.ids = ids;
    a.n_tok = static_cast<int>(n_tok);
    a.top_k = static_cast<int>(top_k);
    const DeviceInfo dv = device_info();
    a.cus = dv.cus;
    a.lds_per_cu = dv.lds_per_cu;
    a.y = gu;
    a.err = reinterpret_cast<int*>(b);
    a.n_ff = static_cast<int>(n_ff);
    a.hq = static_cast<uint8_t*>(hq);
    a.h_off_d = static_cast<int64_t>(qmv_act_offset_d(rows, n_ff));
    a.h_off_s = static_cast<int64_t>(qmv_act_offset_s(rows, n_ff));
    hipError_t e = launch_moe_gate_up_swiglu(a, static_cast<hipStream_t>(stream));
    return hip_status(e);
  }
  // two launches: the routed gate+up into gu (or the workspace's per-slot
  // area, which an unweighted call leaves unused), then SwiGLU + Q8
  float* y = gu != nullptr ? gu : reinterpret_cast<float*>(b + kMoePartOffset);
  st = moe_run(type, w, n_experts, 2 * n_ff, k, xq, 0, ids, nullptr, n_tok, top_k, y, ws, stream);
  if (st != QMV_OK) return st;
  return qmv_swiglu_quantize(y, 2 * n_ff, rows, n_ff, hq, nullptr, stream);
}

// ------------------------------------------------------ no-allocation MoE
// The workspace of qmv_moe_matvec_noalloc: a device array of this library,
// one copy per GPU, alive until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host it only names the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device.
// Nothing in it has to start at zero: every call writes the dropped-slot
// word and the per-slot outputs it reads back.
static __device__ __align__(256) uint8_t scratch[QMV_MOE_NOALLOC_WS_BYTES];

static void* scratch_address(qmv_status* st) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  const hipError_t ed = hipGetDevice(&dev);
  if (ed != hipSuccess || dev < 0 || dev >= 64) {
    *st = ed != hipSuccess ? hip_status(ed) : hip_status(hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || p == nullptr) {
      *st = hip_status(es != hipSuccess ? es : hipErrorInvalidSymbol);
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

QMV_API qmv_status qmv_moe_matvec_noalloc(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows,
                                          int64_t k, const void* xq, int x_per_slot, const int32_t* ids,
                                          const float* route_w, int64_t n_tok, int64_t top_k, float* y,
                                          void* stream) {
  qmv_status st = moe_check(type, w, n_experts, n_rows, k, xq, x_per_slot, ids, route_w, n_tok, top_k, y);
  if (st != QMV_OK) return st;
  if (qmv_moe_workspace_bytes(type, n_experts, n_rows, k, n_tok, top_k) > QMV_MOE_NOALLOC_WS_BYTES)
    return QMV_ERR_WORKSPACE;
  void* ws = scratch_address(&st);
  if (ws == nullptr) return st;
  return moe_run(type, w, n_experts, n_rows, k, xq, x_per_slot, ids, route_w, n_tok, top_k, y, ws, stream);
}

QMV_API qmv_status qmv_moe_block_dots(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows, int64_t k,
                                      const void* xq, int x_per_slot, const int32_t* ids, int64_t n_tok,
                                      int64_t top_k, int64_t slot_rows, int32_t* out, void* ws, size_t ws_bytes,
                                      void* stream) {
  qmv_status st = check_weights(type, w, n_rows, k);
  if (st != QMV_OK) return st;
  if (xq == nullptr || ids == nullptr || out == nullptr || ws == nullptr || n_tok < 1 || top_k < 1 ||
      n_experts < 1 || (x_per_slot != 0 && x_per_slot != 1) || (slot_rows != 0 && slot_rows != 4 && slot_rows != 8))
    return QMV_ERR_INVALID_ARG;
  if (n_tok > QMV_MAX_MOE_TOKENS || top_k > QMV_MAX_TOP_K || n_experts > QMV_MAX_EXPERTS ||
      k / 32 > kMoeMaxUnits || n_rows > kMoeMaxRows || !moe_format(type))
    return QMV_ERR_UNSUPPORTED;
  if (n_experts * n_rows > INT32_MAX || n_tok * top_k * n_rows * (k / 32) > INT32_MAX / 2)
    return QMV_ERR_UNSUPPORTED;
  if (!aligned(xq, 256) || !aligned(ids, 4) || !aligned(out, 4) || !aligned(ws, 256)) return QMV_ERR_MISALIGNED;
  if (ws_bytes < qmv_moe_workspace_bytes(type, n_experts, n_rows, k, n_tok, top_k)) return QMV_ERR_WORKSPACE;
  const int64_t x_rows = x_per_slot ? n_tok * top_k : n_tok;
  MoeLaunch a{};
  a.fmt = type;
  a.w = static_cast<const uint8_t*>(w);
  a.row_bytes = static_cast<int64_t>(qmv_row_bytes(type, k));
  a.n_experts = static_cast<int>(n_experts);
  a.n_rows = static_cast<int>(n_rows);
  a.units = static_cast<int>(k / 32);
  a.x = act_view(xq, x_rows, k);
  a.x_rows = static_cast<int>(x_rows);
  a.x_per_slot = x_per_slot;
  a.ids = ids;
  a.rw = nullptr;
  a.n_tok = static_cast<int>(n_tok);
  a.top_k = static_cast<int>(top_k);
  a.y = nullptr;
  const DeviceInfo dv = device_info();
  a.cus = dv.cus;
  a.lds_per_cu = dv.lds_per_cu;
  uint8_t* b = static_cast<uint8_t*>(ws);
  a.err = reinterpret_cast<int*>(b);
  a.part = reinterpret_cast<float*>(b + kMoePartOffset);
  a.dots = out;
  // the slot rows per group the automatic choice stages: 4 up to 16 tokens, 8 beyond
  const int tm = slot_rows != 0 ? static_cast<int>(slot_rows) : (n_tok <= 16 ? 4 : 8);
  hipError_t e = launch_moe_mx_dots(a, tm, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return QMV_ERR_UNSUPPORTED;  // the staged rows do not fit in LDS
  return hip_status(e);
}
