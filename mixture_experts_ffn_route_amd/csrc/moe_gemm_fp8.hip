// FP8 e4m3 block-scale grouped GEMMs of the MoE layer on gfx950 MFMA.
//
// FC1: for each sorted route row p (expert e, token t)
//   gu[p, n] = sum_kb sx[t, kb] * s13[e, n/128, kb] * sum_{k in kb} xq[t, k] * w13[e, n, k]
//   h = silu(gate) * up, then per 1x128 block of h: s = amax/448, q = RNE_sat(h/s)
// FC2: y[p, n] = sum_kb sh[p, kb] * s2[e, n/128, kb] * sum_{k in kb} hq[p, k] * w2[e, n, k]  -> bf16
//
// These are the "FC1 with fused SwiGLU + 1x128 quantization" and "FC2" steps
// of the forward pipeline in "feat(moe_ep): add SM90 push FP8 mega-MoE backend
// for Hopper" (flashinfer PR #4069, Description), with the DeepSeek-style FP8
// block scaling (128x128 weight scales, 1x128 activation scales) of its
// Limitations.
//
// Design (CDNA4):
//  * One K-block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4.  Its FP32
//    result is promoted into the accumulator with the product of the row's
//    activation scale and the weight block's scale (one FMA per output per
//    K-block), so no FP8 operand is ever rescaled.
//  * Workgroup tile: BM rows x 256 weight rows, 4 waves as 2 (rows) x 2
//    (columns).  FC1's 256 weight rows are the gate and up rows of one
//    128-wide block of h, so the SwiGLU and the 1x128 amax of the epilogue see
//    whole blocks.  FC2's are two 128-row blocks of H.
//  * K-blocks are staged global -> registers -> LDS, double buffered, with
//    16-byte chunks XOR-swizzled by row so MFMA operand reads are conflict
//    free.  FC1 gathers its activation rows by token (one staged row per
//    token: deduplicated staging).
//  * Persistent workgroups: the (row tile, column tile) space is split into
//    eight contiguous ranges, one per XCD (workgroup i runs on XCD i % 8), and
//    neighbouring tiles on an XCD share activation rows and weight columns in
//    its L2.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 256;         // weight rows per tile
constexpr int kKB = 128;         // bytes (= e4m3 elements) per K-block
constexpr int kGroupM = 4;       // row tiles per XCD-local group

__device__ __forceinline__ int swz(int row, int chunk) { return row * kKB + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int c0) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + swz(row, c0));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + swz(row, c0 + 1));
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

template <int BM, bool FC1>
struct GemmTile {
  static constexpr int WM = BM / 2;          // rows per wave
  static constexpr int RB = WM / 16;         // 16-row MFMA blocks per wave
  static constexpr int CB = 8;               // 16-col MFMA blocks per wave (4 per 128-block)
  static constexpr int A_CHUNKS = BM * 8 / kThreads;   // 16-byte A chunks per thread per K-block
  static constexpr int B_CHUNKS = kBN * 8 / kThreads;  // 8
  static constexpr int A_BYTES = BM * kKB;
  static constexpr int B_BYTES = kBN * kKB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + BM * 4;
  static constexpr int OUT_BYTES = FC1 ? (BM * 128 + BM * 4 * 3) : (BM * kBN * 2);
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > OUT_BYTES) ? 2 * STAGE_BYTES : OUT_BYTES;
};

template <int BM, bool FC1>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(GemmArgs a) {
  using G = GemmTile<BM, FC1>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int kbs = a.k_dim / kKB;                 // K-blocks
  const int nblk_w = a.n_rows / 128;             // 128-row weight blocks per expert
  const int total_m = (int)a.hdr[kHdrMTiles];
  const int64_t total = (int64_t)total_m * a.n_tiles;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int per_xcd = gridDim.x >> 3;
  const int64_t v_begin = total * xcd / 8, v_end = total * (xcd + 1) / 8;

  for (int64_t v = v_begin + slot; v < v_end; v += per_xcd) {
    // ---- tile coordinates ------------------------------------------------
    const int64_t group = v / ((int64_t)kGroupM * a.n_tiles);
    const int64_t rem = v - group * kGroupM * a.n_tiles;
    const int m0 = (int)(group * kGroupM);
    const int gm = min(kGroupM, total_m - m0);
    const int nt = (int)(rem / gm);
    const int mt = m0 + (int)(rem % gm);
    const int e = a.tiles[2 * mt];
    const int p0 = a.tiles[2 * mt + 1];
    const int rows_valid = min(BM, a.offsets[e + 1] - p0);

    // weight blocks of this column tile
    int nb0, nb1;
    if (FC1) {
      nb0 = nt;                       // gate block
      nb1 = a.inter / 128 + nt;       // up block
    } else {
      nb0 = 2 * nt;
      nb1 = min(2 * nt + 1, nblk_w - 1);
    }

    // ---- per-thread source addresses ------------------------------------
    const uint8_t* a_src[G::A_CHUNKS];
#pragma unroll
    for (int i = 0; i < G::A_CHUNKS; ++i) {
      const int q = tid + i * kThreads;
      const int row = q >> 3, c = q & 7;
      const int p = p0 + min(row, rows_valid - 1);
      int64_t src = p;
      if (a.a_mode == 1) src = a.sorted_route[p] / a.top_k;
      else if (a.a_mode == 2) src = a.sorted_route[p];
      a_src[i] = a.a + src * a.k_dim + c * 16;
    }
    const float* s_src = nullptr;
    if (tid < BM) {
      const int p = p0 + min(tid, rows_valid - 1);
      int64_t src = p;
      if (a.a_mode == 1) src = a.sorted_route[p] / a.top_k;
      else if (a.a_mode == 2) src = a.sorted_route[p];
      s_src = a.a_scale + src * kbs;
    }
    const uint8_t* b_src[G::B_CHUNKS];
#pragma unroll
    for (int i = 0; i < G::B_CHUNKS; ++i) {
      const int q = tid + i * kThreads;
      const int brow = q >> 3, c = q & 7;
      const int blk = brow < 128 ? nb0 : nb1;
      const int wrow = blk * 128 + (brow & 127);
      b_src[i] = a.w + ((int64_t)e * a.n_rows + wrow) * a.k_dim + c * 16;
    }
    const float* ws0 = a.w_scale + ((int64_t)e * nblk_w + nb0) * kbs;
    const float* ws1 = a.w_scale + ((int64_t)e * nblk_w + nb1) * kbs;

    // ---- main loop --------------------------------------------------------
    v4f acc[G::RB][G::CB];
#pragma unroll
    for (int rb = 0; rb < G::RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < G::CB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[G::A_CHUNKS], rb_[G::B_CHUNKS];
    float rsx = 0.f;
#define MOE_GLOAD(KB)                                                                        \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < G::A_CHUNKS; ++i)                                  \
        ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + (KB) * kKB);                      \
    _Pragma("unroll") for (int i = 0; i < G::B_CHUNKS; ++i)                                  \
        rb_[i] = *reinterpret_cast<const u32x4*>(b_src[i] + (KB) * kKB);                     \
    if (tid < BM) rsx = s_src[(KB)];                                                         \
  } while (0)
#define MOE_LSTORE(STAGE)                                                                    \
  do {                                                                                       \
    uint8_t* As_ = smem + (STAGE) * G::STAGE_BYTES;                                          \
    uint8_t* Bs_ = As_ + G::A_BYTES;                                                         \
    float* Ss_ = reinterpret_cast<float*>(Bs_ + G::B_BYTES);                                 \
    _Pragma("unroll") for (int i = 0; i < G::A_CHUNKS; ++i) {                                \
      const int q = tid + i * kThreads;                                                      \
      *reinterpret_cast<u32x4*>(As_ + swz(q >> 3, q & 7)) = ra[i];                           \
    }                                                                                        \
    _Pragma("unroll") for (int i = 0; i < G::B_CHUNKS; ++i) {                                \
      const int q = tid + i * kThreads;                                                      \
      *reinterpret_cast<u32x4*>(Bs_ + swz(q >> 3, q & 7)) = rb_[i];                          \
    }                                                                                        \
    if (tid < BM) Ss_[tid] = rsx;                                                            \
  } while (0)

    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
    const int c0 = (lane >> 4) * 2;
    for (int kb = 0; kb < kbs; ++kb) {
      const int st = kb & 1;
      const float sw0 = ws0[kb], sw1 = ws1[kb];
      if (kb + 1 < kbs) MOE_GLOAD(kb + 1);
      const uint8_t* As = smem + st * G::STAGE_BYTES;
      const uint8_t* Bs = As + G::A_BYTES;
      const float* Ss = reinterpret_cast<const float*>(Bs + G::B_BYTES);
      v8i af[G::RB];
      float sxa[G::RB][4], sxb[G::RB][4];
#pragma unroll
      for (int rb = 0; rb < G::RB; ++rb) {
        af[rb] = lds_frag(As, wm * G::WM + rb * 16 + (lane & 15), c0);
        const v4f sx = *reinterpret_cast<const v4f*>(Ss + wm * G::WM + rb * 16 + (lane >> 4) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sxa[rb][i] = sx[i] * sw0;
          sxb[rb][i] = sx[i] * sw1;
        }
      }
#pragma unroll
      for (int cb = 0; cb < G::CB; ++cb) {
        const int col = (cb < 4 ? 0 : 128) + wn * 64 + (cb & 3) * 16 + (lane & 15);
        const v8i bf = lds_frag(Bs, col, c0);
#pragma unroll
        for (int rb = 0; rb < G::RB; ++rb) {
          const v4f p = mfma_fp8(af[rb], bf);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][cb][i] = fmaf(p[i], cb < 4 ? sxa[rb][i] : sxb[rb][i], acc[rb][cb][i]);
        }
      }
      if (kb + 1 < kbs) MOE_LSTORE(st ^ 1);
      __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    if (FC1) {
      // h = silu(gate) * up for this lane's 4 columns of each row
      float* red = reinterpret_cast<float*>(smem + BM * 128);   // [2][BM] partial amax
      float* sca = red + 2 * BM;                                // [BM] scales
      float h[G::RB][4][4];
#pragma unroll
      for (int rb = 0; rb < G::RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float m = 0.f;
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const float g = acc[rb][c4][i], u = acc[rb][c4 + 4][i];
            const float hv = g / (1.0f + expf(-g)) * u;
            h[rb][c4][i] = hv;
            m = fmaxf(m, fabsf(hv));
          }
          m = group_max<16>(m);
          if ((lane & 15) == 0) red[wn * BM + wm * G::WM + rb * 16 + (lane >> 4) * 4 + i] = m;
        }
      __syncthreads();
      uint8_t* out = smem;  // [BM][128] codes
#pragma unroll
      for (int rb = 0; rb < G::RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * G::WM + rb * 16 + (lane >> 4) * 4 + i;
          const float amax = fmaxf(red[row], red[BM + row]);
          const float s = amax / kE4m3Max;
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const float q = s == 0.f ? 0.f : h[rb][c4][i] / s;
            const int code = s == 0.f ? 0 : (cvt2_e4m3(q, 0.f, 0, false) & 0xff);
            out[row * 128 + wn * 64 + c4 * 16 + (lane & 15)] = (uint8_t)code;
          }
          if (wn == 0 && (lane & 15) == 0) sca[row] = s;
        }
      __syncthreads();
      const int ikb = a.inter / 128;
      for (int q = tid; q < BM * 8; q += kThreads) {
        const int row = q >> 3, c = q & 7;
        if (row < rows_valid)
          *reinterpret_cast<u32x4*>(a.hq + (int64_t)(p0 + row) * a.inter + nt * 128 + c * 16) =
              *reinterpret_cast<const u32x4*>(out + row * 128 + c * 16);
      }
      if (tid < rows_valid) a.hs[(int64_t)(p0 + tid) * ikb + nt] = sca[tid];
    } else {
      uint16_t* out = reinterpret_cast<uint16_t*>(smem);  // [BM][256] bf16
#pragma unroll
      for (int rb = 0; rb < G::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < G::CB; ++cb) {
          const int col = (cb < 4 ? 0 : 128) + wn * 64 + (cb & 3) * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = wm * G::WM + rb * 16 + (lane >> 4) * 4 + i;
            out[row * kBN + col] = (uint16_t)f32_to_bf16_rne(acc[rb][cb][i]);
          }
        }
      __syncthreads();
      const int n0 = nt * kBN;
      const int ncols = min(kBN, a.n_rows - n0);
      for (int q = tid; q < BM * 32; q += kThreads) {
        const int row = q >> 5, c = (q & 31) * 8;
        if (row < rows_valid && c < ncols)
          *reinterpret_cast<u32x4*>(a.y + (int64_t)(p0 + row) * a.n_rows + n0 + c) =
              *reinterpret_cast<const u32x4*>(out + row * kBN + c);
      }
    }
    __syncthreads();
  }
}

template <int BM, bool FC1>
static int launch_one(const GemmArgs& a, void* stream) {
  hipLaunchKernelGGL((gemm_fp8_kernel<BM, FC1>), dim3(a.grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool FC1>
static int launch_bm(const GemmArgs& a, int block_m, void* stream) {
  switch (block_m) {
    case 32: return launch_one<32, FC1>(a, stream);
    case 64: return launch_one<64, FC1>(a, stream);
    case 128: return launch_one<128, FC1>(a, stream);
  }
  return -1;
}

int launch_fc1(const GemmArgs& a, int block_m, void* stream) { return launch_bm<true>(a, block_m, stream); }
int launch_fc2(const GemmArgs& a, int block_m, void* stream) { return launch_bm<false>(a, block_m, stream); }

template <int BM, bool FC1>
static int occ() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_kernel<BM, FC1>, kThreads, 0) != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

int gemm_max_workgroups_per_cu(int which, int block_m) {
  if (which == 1) {
    switch (block_m) { case 32: return occ<32, true>(); case 64: return occ<64, true>(); default: return occ<128, true>(); }
  }
  switch (block_m) { case 32: return occ<32, false>(); case 64: return occ<64, false>(); default: return occ<128, false>(); }
}

}  // namespace moe
