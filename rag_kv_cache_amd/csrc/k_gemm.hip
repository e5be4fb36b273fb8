// GEMMs of the fusion step: C[M][N] = A[M][K] * B[N][K]^T (B = nn.Linear weight rows) with a
// fused epilogue.  Used for the fresh K/V and Q of the selected rows (RoPE epilogue), the
// o-projection and the FFN down-projection (residual-add epilogue), and the FFN gate/up
// projection (SwiGLU epilogue).
//
// bf16 path: v_mfma_f32_16x16x32_bf16 on gfx950.  Workgroup = 4 wavefronts (2 x 2), tile
// BM x 128 x 64 (BM = 128 or 64), both operands staged through LDS with a 16-byte row pad,
// double-buffered: the next K-slab is fetched into registers while the current one feeds
// the MFMAs.  Rows of A may be gathered through an index list (the selected rows).
// Tiles are assigned XCD-contiguously (see xcd_tile) so that the workgroups reading the
// same weight columns run on one XCD and share its L2.
// Split-K (grid.y > 1) writes fp32 partial tiles; a reduce kernel sums them and applies
// the same epilogue.
//
// MFMA operand layout used (16x16x32, 8 bf16 per lane): lane l supplies row (l & 15) of A
// and column (l & 15) of B, both with the same 8 reduction slots (l >> 4) * 8 .. + 7; lane l
// receives C[4 * (l >> 4) + r][l & 15], r = 0..3.
#include "cb_common.h"
#include "cb_kernels.h"

namespace cb {
namespace {

constexpr int BN = 128;
constexpr int BK = 64;
constexpr int KP = BK + 8;    // LDS row pitch of A/B tiles (bf16 elements)
constexpr int CP = BN + 4;    // LDS row pitch of the staged fp32 C tile

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// Column pair handled by epilogue item c (0..63) of a 128-wide tile.  RoPE rotates pairs
// (i, i + head_dim/2) within each head; the other epilogues use (c, c + 64), which for the
// SwiGLU tile is (gate, up) of the same FFN feature.
__device__ __forceinline__ void epi_cols(int epi, int head_dim, int c, int& c0, int& c1) {
  if (epi == EPI_ROPE) {
    const int half = head_dim >> 1;
    const int hb = c / half, i = c - hb * half;
    c0 = hb * head_dim + i;
    c1 = c0 + half;
  } else {
    c0 = c;
    c1 = c + 64;
  }
}

template <typename TO>
__device__ __forceinline__ void epi_apply(const GemmArgs& g, int m, int n0, int c0, int c1, float v0, float v1) {
  switch (g.epi) {
    case EPI_ROPE: {
      const int n = n0 + c0;
      if (n < g.rope_cols) {
        int p = g.pos[m];
        p = p < 0 ? 0 : (p > g.max_pos ? g.max_pos : p);
        const int half = g.head_dim >> 1;
        const float2 t = g.rope[(long)p * half + (n % g.head_dim)];
        const float y0 = v0 * t.x - v1 * t.y;
        const float y1 = v1 * t.x + v0 * t.y;
        v0 = y0;
        v1 = y1;
      }
      TO* o = (TO*)g.out + (long)m * g.ldo + n0;
      Elem<TO>::st(o + c0, v0);
      Elem<TO>::st(o + c1, v1);
      break;
    }
    case EPI_SWIGLU: {
      TO* o = (TO*)g.out + (long)m * g.ldo + (n0 >> 1);
      Elem<TO>::st(o + c0, silu(v0) * v1);
      break;
    }
    case EPI_RESID: {
      const long rr = g.resid_rows ? (long)g.resid_rows[m] : (long)m;
      const float* r = g.resid + rr * g.ldr + n0;
      float* o = (float*)g.out + (long)m * g.ldo + n0;
      o[c0] = r[c0] + v0;
      o[c1] = r[c1] + v1;
      break;
    }
    default: {
      TO* o = (TO*)g.out + (long)m * g.ldo + n0;
      Elem<TO>::st(o + c0, v0);
      Elem<TO>::st(o + c1, v1);
    }
  }
}

// Weight row feeding virtual column n of tile tn.
__device__ __forceinline__ long b_row(const GemmArgs& g, int tn, int r) {
  if (g.swiglu_ffn > 0) return r < 64 ? (long)tn * 64 + r : (long)g.swiglu_ffn + (long)tn * 64 + (r - 64);
  return (long)tn * BN + r;
}

// Apply the epilogue to a BM x 128 fp32 tile staged in LDS (pitch CP).
template <typename TO, int BMr, int NT>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const float* Cs, int m0, int n0) {
  const int c = threadIdx.x & 63;
  int c0, c1;
  epi_cols(g.epi, g.head_dim, c, c0, c1);
  for (int rr = threadIdx.x >> 6; rr < BMr; rr += NT / 64) {
    const int m = m0 + rr;
    if (m >= g.M) break;
    epi_apply<TO>(g, m, n0, c0, c1, Cs[rr * CP + c0], Cs[rr * CP + c1]);
  }
}

template <int BM>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WTM = BM / 2;        // wave tile rows (2 x 2 wavefronts)
  constexpr int FM = WTM / 16;       // 16-row MFMA blocks per wave
  constexpr int FN = 4;              // 16-col MFMA blocks per wave (64 cols)
  constexpr int A_PT = BM * BK / 8 / 256;
  constexpr int B_PT = BN * BK / 8 / 256;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* As = reinterpret_cast<bf16_t*>(smem);  // [2][BM][KP]
  bf16_t* Bs = As + 2 * BM * KP;                 // [2][BN][KP]

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
  if (tile < 0) return;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_len = g.K / g.splits;
  const int kb = blockIdx.y * k_len, ke = kb + k_len;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);
  const bf16_t* B = reinterpret_cast<const bf16_t*>(g.B);

  const bf16_t* a_src[A_PT];
  bool a_ok[A_PT];
  int a_off[A_PT];
#pragma unroll
  for (int i = 0; i < A_PT; ++i) {
    const int v = tid + 256 * i, r = v >> 3, c = (v & 7) * 8;
    const int m = m0 + r;
    a_ok[i] = m < g.M;
    const long row = a_ok[i] ? (g.a_rows ? (long)g.a_rows[m] : (long)m) : 0;
    a_src[i] = A + row * g.lda + c;
    a_off[i] = r * KP + c;
  }
  const bf16_t* b_src[B_PT];
  int b_off[B_PT];
#pragma unroll
  for (int i = 0; i < B_PT; ++i) {
    const int v = tid + 256 * i, r = v >> 3, c = (v & 7) * 8;
    b_src[i] = B + b_row(g, tn, r) * g.ldb + c;
    b_off[i] = r * KP + c;
  }

  uint4 ra[A_PT], rb[B_PT];
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < B_PT; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + k);
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) *reinterpret_cast<uint4*>(As + buf * BM * KP + a_off[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PT; ++i) *reinterpret_cast<uint4*>(Bs + buf * BN * KP + b_off[i]) = rb[i];
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(kb);
  swrite(0);
  __syncthreads();
  int buf = 0;
  for (int k = kb; k < ke; k += BK) {
    const bool more = k + BK < ke;
    if (more) gload(k + BK);
    const bf16_t* Ab = As + buf * BM * KP + (wm * WTM + (lane & 15)) * KP + (lane >> 4) * 8;
    const bf16_t* Bb = Bs + buf * BN * KP + (wn * 64 + (lane & 15)) * KP + (lane >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(Ab + i * 16 * KP + ks * 32);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bb + j * 16 * KP + ks * 32);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) swrite(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  if (g.splits > 1) {  // fp32 partial tile straight from registers
    float* P = g.partial + (long)blockIdx.y * g.M * g.N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * WTM + i * 16 + (lane >> 4) * 4 + r;
          const int n = n0 + wn * 64 + j * 16 + (lane & 15);
          if (m < g.M) P[(long)m * g.N + n] = acc[i][j][r];
        }
    return;
  }
  float* Cs = reinterpret_cast<float*>(smem);  // [BM][CP]; A/B tiles are no longer read
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(wm * WTM + i * 16 + (lane >> 4) * 4 + r) * CP + wn * 64 + j * 16 + (lane & 15)] = acc[i][j][r];
  __syncthreads();
  tile_epilogue<bf16_t, BM, 256>(g, Cs, m0, n0);
}

// Sum split-K partials and apply the epilogue.  grid = (ceil(M/4), N/128), 256 threads:
// 4 rows x 64 column pairs.
template <typename TO>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = blockIdx.y * BN;
  if (m >= g.M) return;
  int c0, c1;
  epi_cols(g.epi, g.head_dim, threadIdx.x & 63, c0, c1);
  float v0 = 0.f, v1 = 0.f;
  const long stride = (long)g.M * g.N;
  const float* p = g.partial + (long)m * g.N + n0;
  for (int s = 0; s < g.splits; ++s) {
    v0 += p[s * stride + c0];
    v1 += p[s * stride + c1];
  }
  epi_apply<TO>(g, m, n0, c0, c1, v0, v1);
}

// fp32 path (correctness configurations): tile 64 x 128 x 16 on the vector ALUs, each
// thread 4 rows x 8 columns, operands through LDS, same epilogues.
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int FBM = 64, FBK = 16;
  __shared__ __align__(16) float smem[FBM * CP];  // staged C tile; also holds the A/B tiles
  float* As = smem;                // [FBK][FBM]
  float* Bs = smem + FBK * FBM;    // [FBK][BN]
  const int tiles_m = (g.M + FBM - 1) / FBM;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * FBM, n0 = tn * BN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* A = reinterpret_cast<const float*>(g.A);
  const float* B = reinterpret_cast<const float*>(g.B);
  float acc[4][8] = {};
  // A tile: 64 rows x 16 k = 256 float4, one per thread.  B tile: 128 x 16 = 512 float4.
  const int ar = tid >> 2, ak = (tid & 3) * 4;
  const int am = m0 + ar;
  const bool a_ok = am < g.M;
  const float* a_src = A + (a_ok ? (g.a_rows ? (long)g.a_rows[am] : (long)am) : 0) * g.lda + ak;
  const int br = tid >> 2, bk = (tid & 3) * 4;
  const float* b_src0 = B + b_row(g, tn, br) * g.ldb + bk;
  const float* b_src1 = B + b_row(g, tn, br + 64) * g.ldb + bk;
  for (int k = 0; k < g.K; k += FBK) {
    const float4 av = a_ok ? *reinterpret_cast<const float4*>(a_src + k) : make_float4(0, 0, 0, 0);
    const float4 b0 = *reinterpret_cast<const float4*>(b_src0 + k);
    const float4 b1 = *reinterpret_cast<const float4*>(b_src1 + k);
    As[(ak + 0) * FBM + ar] = av.x; As[(ak + 1) * FBM + ar] = av.y;
    As[(ak + 2) * FBM + ar] = av.z; As[(ak + 3) * FBM + ar] = av.w;
    Bs[(bk + 0) * BN + br] = b0.x; Bs[(bk + 1) * BN + br] = b0.y;
    Bs[(bk + 2) * BN + br] = b0.z; Bs[(bk + 3) * BN + br] = b0.w;
    Bs[(bk + 0) * BN + br + 64] = b1.x; Bs[(bk + 1) * BN + br + 64] = b1.y;
    Bs[(bk + 2) * BN + br + 64] = b1.z; Bs[(bk + 3) * BN + br + 64] = b1.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      const float4 a4 = *reinterpret_cast<const float4*>(As + kk * FBM + ty * 4);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float b = Bs[kk * BN + tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = fmaf(a[i], b, acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) smem[(ty * 4 + i) * CP + tx + 16 * j] = acc[i][j];
  __syncthreads();
  tile_epilogue<float, FBM, 256>(g, smem, m0, n0);
}

template <int BM>
constexpr int bf16_lds_bytes() {
  return (2 * (BM + BN) * KP * 2) > (BM * CP * 4) ? (2 * (BM + BN) * KP * 2) : (BM * CP * 4);
}

template <int BM>
hipError_t launch_bf16(const GemmArgs& g, hipStream_t s) {
  static bool attr_set = false;
  constexpr int lds = bf16_lds_bytes<BM>();
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<BM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN);
  const int grid_x = 8 * ((tiles + 7) / 8);
  hipLaunchKernelGGL(gemm_bf16_kernel<BM>, dim3(grid_x, g.splits), dim3(256), lds, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int tiles128 = ((g.M + 127) / 128) * (g.N / BN);
  hipError_t e = (tiles128 >= 240) ? launch_bf16<128>(g, s) : launch_bf16<64>(g, s);
  if (e != hipSuccess || g.splits <= 1) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, dim3((g.M + 3) / 4, g.N / BN), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int tiles = ((g.M + 63) / 64) * (g.N / BN);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace cb
