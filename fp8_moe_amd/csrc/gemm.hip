// Host side of the grouped expert GEMMs: parameter setup and dispatch to the
// kernel instantiations (the kernel is in gemm_kernel.h).
#include "gemm_kernel.h"

namespace b12x {

#define B12X_GEMM_ALL(X)                                   \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE_SILU)          \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE_RELU2)         \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE_DOWN)          \
  X(B12X_WEIGHT_NVFP4, kActF16NvRt, MODE_SILU)             \
  X(B12X_WEIGHT_NVFP4, kActF16NvRt, MODE_RELU2)            \
  X(B12X_WEIGHT_NVFP4, kActF16Rt, MODE_SILU)               \
  X(B12X_WEIGHT_NVFP4, kActF16Rt, MODE_RELU2)              \
  X(B12X_WEIGHT_NVFP4, kActF16, MODE_SILU)                 \
  X(B12X_WEIGHT_NVFP4, kActF16, MODE_RELU2)                \
  X(B12X_WEIGHT_NVFP4, kActRt, MODE_SILU)                  \
  X(B12X_WEIGHT_NVFP4, kActRt, MODE_RELU2)                 \
  X(B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE_SILU)           \
  X(B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE_RELU2)          \
  X(B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE_DOWN)           \
  X(B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE_DENSE)          \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE_SILU)           \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE_RELU2)          \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE_DOWN)           \
  X(B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE_DENSE)
B12X_GEMM_ALL(B12X_GEMM_EXTERN)

static int g_cu_count[64];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!g_cu_count[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

template <int MODE>
static int dispatch(const BindingImpl& b, const GemmParams& p, int64_t max_work, hipStream_t s) {
  const bool nv = b.wfmt == B12X_WEIGHT_NVFP4, a8 = a8_native(b.wfmt, b.afmt);
  if (a8) return launch_gemm_t<B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE>(p, max_work, s);
  if constexpr (MODE != MODE_DOWN) {
    // the scaled f16 copy of a (of its MXFP8 round trips with MXFP8 activations), else the
    // bf16 copy of the round trips
    if (p.a_exp && a4_nv(b.afmt)) return launch_gemm_t<B12X_WEIGHT_NVFP4, kActF16NvRt, MODE>(p, max_work, s);
    if (p.a_exp && a8_bf16(b.wfmt, b.afmt)) return launch_gemm_t<B12X_WEIGHT_NVFP4, kActF16Rt, MODE>(p, max_work, s);
    if (p.a_exp) return launch_gemm_t<B12X_WEIGHT_NVFP4, kActF16, MODE>(p, max_work, s);
    if (a8_bf16(b.wfmt, b.afmt)) return launch_gemm_t<B12X_WEIGHT_NVFP4, kActRt, MODE>(p, max_work, s);
  }
  if (nv) return launch_gemm_t<B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE>(p, max_work, s);
  return launch_gemm_t<B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE>(p, max_work, s);
}

int launch_gemm1(const BindingImpl& b, hipStream_t s) {
  GemmParams p = {};
  p.lv = b.live();
  p.oai = b.oai;
  const bool a8 = a8_native(b.wfmt, b.afmt);
  p.tiles = b.tiles;
  p.ntiles = b.ntiles;
  p.max_tiles = (int)b.max_tiles;
  p.max_rows = (int)b.max_rows;
  p.E = b.E;
  p.n_ntiles = (int)((b.nf13 + 4 * kGemmNFW - 1) / (4 * kGemmNFW));
  p.a16 = b.a;
  p.a8 = b.xq;
  p.as = b.xs;
  p.a_stride = a8 ? b.Hp : b.a_stride;
  p.as_stride = b.Hp / 32;
  p.a_bytes = a8 ? b.T * b.Hp : b.T * b.a_stride * 2;
  p.as_bytes = a8 ? b.T * (b.Hp / 32) : 0;
  if (b.a_f16) {  // NVFP4 x bf16: the scaled f16 copy of a and its row exponents
    p.a16 = (const uint16_t*)b.xq;
    p.a_stride = b.Hp;
    p.a_bytes = b.T * b.Hp * 2;
    p.a_exp = (const int32_t*)b.xs;
  }
  // (NVFP4 x MXFP8 and NVFP4 x NVFP4 take the same route: the copy then holds a's round trips)
  if (a4_nv(b.afmt)) {
    p.aglobal = b.a13_global;  // x's activation scale, one value
    p.aglobal_per_expert = 0;
    p.hglobal = b.a2_global;   // h is requantized against its expert's scale
  }
  p.sorted = b.sorted;
  p.k_top = b.k;
  p.n_pairs = b.T * b.k;
  p.K = b.H;
  p.KF = (int)b.kf13;
  p.bcodes = b.w13_codes;
  p.bscales = b.w13_scales;
  p.bglobal = b.w13_global;
  p.b_codes_expert = b.nf13 * b.kf13 * kFragBytes;
  p.b_scales_expert = b.nf13 * b.kfs13 * kScaleGroupBytes;
  p.NF = (int)b.nf13;
  p.KFS = (int)b.kfs13;
  p.h16 = (uint16_t*)b.h;
  p.h8 = (uint8_t*)b.h;
  p.hs = b.hs;
  p.h_stride = b.Ip;
  p.hs_stride = b.Ip / 32;
  const int64_t max_work = b.max_tiles * p.n_ntiles;
  return b.gated ? dispatch<MODE_SILU>(b, p, max_work, s) : dispatch<MODE_RELU2>(b, p, max_work, s);
}

int launch_gemm2(const BindingImpl& b, hipStream_t s) {
  GemmParams p = {};
  p.lv = b.live();
  const bool a8 = a8_native(b.wfmt, b.afmt);  // else h is bf16
  p.tiles = b.tiles;
  p.ntiles = b.ntiles;
  p.max_tiles = (int)b.max_tiles;
  p.max_rows = (int)b.max_rows;
  p.E = b.E;
  p.n_ntiles = (int)((b.nf2 + 4 * kGemmNFW - 1) / (4 * kGemmNFW));
  p.a16 = (const uint16_t*)b.h;
  p.a8 = (const uint8_t*)b.h;
  p.as = b.hs;
  p.a_stride = b.Ip;
  p.as_stride = b.Ip / 32;
  p.a_bytes = b.max_rows * b.Ip * (a8 ? 1 : 2);
  p.as_bytes = a8 ? b.max_rows * (b.Ip / 32) : 0;
  p.sorted = nullptr;
  p.k_top = b.k;
  p.K = b.I;
  p.KF = (int)b.kf2;
  p.bcodes = b.w2_codes;
  p.bscales = b.w2_scales;
  p.bglobal = b.w2_global;
  p.b_codes_expert = b.nf2 * b.kf2 * kFragBytes;
  p.b_scales_expert = b.nf2 * b.kfs2 * kScaleGroupBytes;
  p.NF = (int)b.nf2;
  p.KFS = (int)b.kfs2;
  p.out16 = b.y16;
  p.out_stride = b.H;
  if (a4_nv(b.afmt)) {  // h's activation scale, one per expert
    p.aglobal = b.a2_global;
    p.aglobal_per_expert = 1;
  }
  const int64_t max_work = b.max_tiles * p.n_ntiles;
  return dispatch<MODE_DOWN>(b, p, max_work, s);
}

// Dense GEMM out[m, n] = bf16(x[m, :] . W[n, :] * g): the grouped GEMM's down
// path with one weight matrix and the rows of x in tiles of kTileRows.
int launch_dense_mm(const uint16_t* x, int64_t m, int64_t x_stride, const uint8_t* w, const MatrixLayout& l,
                    int wfmt, const float* global_scale, uint16_t* out, int64_t out_stride, hipStream_t s) {
  GemmParams p = {};
  p.dense_m = m;
  p.max_rows = (int)m;
  p.max_tiles = (int)((m + kTileRows - 1) / kTileRows);
  p.E = 1;
  p.n_ntiles = (int)((l.nf + 4 * kGemmNFW - 1) / (4 * kGemmNFW));
  p.a16 = x;
  p.a_stride = x_stride;
  p.a_bytes = m * x_stride * 2;
  p.K = l.k;
  p.KF = (int)l.kf;
  p.bcodes = w;
  p.bscales = w + dense_scales_offset(l);
  p.bglobal = global_scale;
  p.b_codes_expert = (int64_t)l.codes_per_expert;
  p.b_scales_expert = (int64_t)l.scales_per_expert;
  p.NF = (int)l.nf;
  p.KFS = (int)l.kfs;
  p.out16 = out;
  p.out_stride = out_stride;
  const int64_t max_work = (int64_t)p.max_tiles * p.n_ntiles;
  if (wfmt == B12X_WEIGHT_NVFP4) return launch_gemm_t<B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE_DENSE>(p, max_work, s);
  return launch_gemm_t<B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE_DENSE>(p, max_work, s);
}

}  // namespace b12x
