// Sparse-query causal GQA attention (CacheBlend review: the selected tokens' queries attend,
// under the causal mask, to all available K/V; tokens that were not recomputed stay keys).
//
// Query rows are the kept rows of the layer (ascending positions qpos); keys are every fused
// K/V row 0 .. qpos[row].  bf16 path (head_dim 128):
//   workgroup = 16 consecutive query rows x all G query heads of one KV head (one
//   wavefront per query head, so the K/V tile in LDS serves the whole GQA group);
//   64-key tiles: K stored row-major, V stored transposed (V^T[dim][key]) in LDS;
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K as the A operand, the wave's Q rows held
//   in registers as the B operand), so every lane owns one query row's scores: lane l has
//   row (l & 15) and keys 4*(l >> 4) + r of each 16-key block;
//   online softmax in fp32 (exp2 with log2(e)/sqrt(d) folded into the scale), row max and
//   sum over the four lanes of a row by two xor-shuffles;
//   O^T += V^T P^T: P (rounded to bf16) is already in B-operand layout, V^T is read as two
//   8-byte pieces per lane with the matching key order;
//   split-KV: grid.y splits the key range so short query sets still fill the chip; partial
//   (O, max, sum) go to fp32 buffers merged by attn_combine_kernel.
#include "cb_common.h"
#include "cb_kernels.h"

namespace cb {
namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

template <int G>
__global__ __launch_bounds__(64 * G) void attn_bf16_kernel(AttnArgs a) {
  constexpr int DH = 128, BKV = 64, NT = 64 * G;
  constexpr int KSP = DH + 8;   // K tile pitch (bf16)
  constexpr int VSP = BKV + 8;  // V^T tile pitch (bf16)
  __shared__ __align__(16) bf16_t Ks[BKV * KSP];
  __shared__ __align__(16) bf16_t Vt[DH * VSP];

  const int qt = blockIdx.x / a.hkv;
  const int g = blockIdx.x - qt * a.hkv;
  const int split = blockIdx.y;
  const int row0 = qt * 16;
  const int last = min(row0 + 16, a.n_q) - 1;
  const int maxpos = a.qpos[last];
  const int kbeg = split * a.split_len;
  if (kbeg > maxpos) return;
  const int kend = min(min(kbeg + a.split_len, maxpos + 1), a.n_tok);
  const int minpos = a.qpos[row0];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = g * G + wave;
  const int l16 = lane & 15, lg = lane >> 4;
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q);
  const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k);
  const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v);
  const long kv_row = (long)a.hkv * DH;

  const int my_row = row0 + l16;
  const bool row_ok = my_row < a.n_q;
  const int mypos = row_ok ? a.qpos[my_row] : -1;
  bf16x8_t qf[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    if (row_ok)
      qf[ds] = *reinterpret_cast<const bf16x8_t*>(Q + (long)my_row * a.ldq + h * DH + ds * 32 + lg * 8);
    else
      qf[ds] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  float m_i = NEG_INF, l_i = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kt = kbeg; kt < kend; kt += BKV) {
    // K tile: 64 keys x 128 dims, 16-byte vectors, row-major in LDS
    for (int v = tid; v < BKV * DH / 8; v += NT) {
      const int kr = v >> 4, c = (v & 15) * 8;
      const int key = kt + kr;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (key < kend) val = *reinterpret_cast<const uint4*>(Kg + key * kv_row + g * DH + c);
      *reinterpret_cast<uint4*>(Ks + kr * KSP + c) = val;
    }
    // V tile transposed: micro-blocks of 4 keys x 4 dims (four 8-byte loads, four 8-byte stores)
    for (int v = tid; v < (BKV / 4) * (DH / 4); v += NT) {
      const int kb4 = v >> 5, d4 = v & 31;
      uint2 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt + kb4 * 4 + i;
        r[i] = make_uint2(0, 0);
        if (key < kend) r[i] = *reinterpret_cast<const uint2*>(Vg + key * kv_row + g * DH + d4 * 4);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int sh = (d & 1) * 16;
        const uint32_t e0 = ((d < 2 ? r[0].x : r[0].y) >> sh) & 0xffffu;
        const uint32_t e1 = ((d < 2 ? r[1].x : r[1].y) >> sh) & 0xffffu;
        const uint32_t e2 = ((d < 2 ? r[2].x : r[2].y) >> sh) & 0xffffu;
        const uint32_t e3 = ((d < 2 ? r[3].x : r[3].y) >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(Vt + (d4 * 4 + d) * VSP + kb4 * 4) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
      }
    }
    __syncthreads();

    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(Ks + (kb * 16 + l16) * KSP + ds * 32 + lg * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ds], s[kb], 0, 0, 0);
      }
    }
    const bool need_mask = (kt + BKV > kend) || (kt + BKV - 1 > minpos);
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[kb][r] * a.scale_log2;
        if (need_mask) {
          const int key = kt + kb * 16 + lg * 4 + r;
          if (key > mypos || key >= kend) x = NEG_INF;
        }
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_i, mx);
    const bool dead = m_new == NEG_INF;
    const float alpha = dead ? 1.f : exp2f(m_i - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = dead ? 0.f : exp2f(s[kb][r] - m_new);
        s[kb][r] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] *= alpha;

#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pf[r] = __builtin_bit_cast(__bf16, f32_to_bf16(s[2 * ks][r]));
        pf[4 + r] = __builtin_bit_cast(__bf16, f32_to_bf16(s[2 * ks + 1][r]));
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16_t* vp = Vt + (d * 16 + l16) * VSP + ks * 32 + lg * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[d], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!row_ok) return;
  // o[d][r] = O[my_row][d*16 + 4*lg + r]
  if (a.splits == 1) {
    const float inv = l_i > 0.f ? 1.f / l_i : 0.f;
    bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + (long)my_row * a.ldo + h * DH + lg * 4;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w0 = (uint32_t)f32_to_bf16(o[d][0] * inv) | ((uint32_t)f32_to_bf16(o[d][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(o[d][2] * inv) | ((uint32_t)f32_to_bf16(o[d][3] * inv) << 16);
      *reinterpret_cast<uint2*>(out + d * 16) = make_uint2(w0, w1);
    }
  } else {
    const long idx = ((long)split * a.n_q + my_row) * a.hq + h;
    float* po = a.part_o + idx * DH + lg * 4;
#pragma unroll
    for (int d = 0; d < 8; ++d) *reinterpret_cast<float4*>(po + d * 16) = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
    if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + idx * 2) = make_float2(m_i, l_i);
  }
}

// Merge split-KV partials: out = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  Only splits
// whose first key is <= the row's position hold keys of that row.  One thread per
// (row, head, 4 dims).
template <typename TO>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int d4n = a.dh / 4;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.n_q * a.hq * d4n;
  if (idx >= total) return;
  const int row = (int)(idx / ((long)a.hq * d4n));
  const int rem = (int)(idx - (long)row * a.hq * d4n);
  const int h = rem / d4n, d0 = (rem - h * d4n) * 4;
  const int ns = min(a.qpos[row] / a.split_len + 1, a.splits);
  float M = NEG_INF;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[(((long)s * a.n_q + row) * a.hq + h) * 2]);
  float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const long pi = ((long)s * a.n_q + row) * a.hq + h;
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + pi * 2);
    if (ml.x == NEG_INF) continue;
    const float w = exp2f(ml.x - M);
    L += ml.y * w;
    const float4 v = *reinterpret_cast<const float4*>(a.part_o + pi * a.dh + d0);
    acc[0] += v.x * w; acc[1] += v.y * w; acc[2] += v.z * w; acc[3] += v.w * w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  TO* out = reinterpret_cast<TO*>(a.out) + (long)row * a.ldo + h * a.dh + d0;
#pragma unroll
  for (int i = 0; i < 4; ++i) Elem<TO>::st(out + i, acc[i] * inv);
}

// fp32 path (correctness configurations): one thread per (query row, query head), online
// softmax over keys 0 .. qpos[row], head_dim DH in registers.
template <int DH>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_q * a.hq) return;
  const int row = idx / a.hq, h = idx - row * a.hq;
  const int g = h / (a.hq / a.hkv);
  const int kend = min(a.qpos[row] + 1, a.n_tok);
  const float* q = reinterpret_cast<const float*>(a.q) + (long)row * a.ldq + h * DH;
  const float* K = reinterpret_cast<const float*>(a.k) + (long)g * DH;
  const float* V = reinterpret_cast<const float*>(a.v) + (long)g * DH;
  const long kv_row = (long)a.hkv * DH;
  float qr[DH], acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) { qr[d] = q[d]; acc[d] = 0.f; }
  float m = NEG_INF, l = 0.f;
  for (int key = 0; key < kend; ++key) {
    const float* kr = K + key * kv_row;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) s = fmaf(qr[d], kr[d], s);
    s *= a.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
    const float* vr = V + key * kv_row;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, vr[d], acc[d] * alpha);
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* out = reinterpret_cast<float*>(a.out) + (long)row * a.ldo + h * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) out[d] = acc[d] * inv;
}

}  // namespace

hipError_t attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_q <= 0) return hipSuccess;
  const int G = a.hq / a.hkv;
  dim3 grid(((a.n_q + 15) / 16) * a.hkv, a.splits);
  switch (G) {
    case 1: hipLaunchKernelGGL(attn_bf16_kernel<1>, grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_bf16_kernel<2>, grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL(attn_bf16_kernel<6>, grid, dim3(384), 0, s, a); break;
    case 7: hipLaunchKernelGGL(attn_bf16_kernel<7>, grid, dim3(448), 0, s, a); break;
    case 8: hipLaunchKernelGGL(attn_bf16_kernel<8>, grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  const long total = (long)a.n_q * a.hq * (a.dh / 4);
  hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_q <= 0) return hipSuccess;
  const int n = a.n_q * a.hq;
  dim3 grid((n + 127) / 128);
  if (a.dh == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(128), 0, s, a);
  else if (a.dh == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(128), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cb
