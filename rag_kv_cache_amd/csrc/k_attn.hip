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

template <int G, int RB>
__global__ __launch_bounds__(64 * G) void attn_bf16_kernel(AttnArgs a) {
  constexpr int DH = 128, BKV = 64, NT = 64 * G, BQ = 16 * RB;
  constexpr int KP = DH + 8;    // K tile pitch (272 B): 16-byte fragment reads of 16 rows hit disjoint banks
  constexpr int VP = DH + 16;   // V tile pitch (288 B): transpose reads of 8 rows x 32 B hit disjoint banks
  constexpr int NVEC = 2 * BKV * DH / 8;   // 16-byte vectors per K+V tile
  constexpr int L_PT = (NVEC + NT - 1) / NT;
  __shared__ __align__(16) bf16_t Ks[2][BKV * KP];
  __shared__ __align__(16) bf16_t Vs[2][BKV * VP];

  const int qt = blockIdx.x / a.hkv;
  const int g = blockIdx.x - qt * a.hkv;
  const int split = blockIdx.y;
  const int row0 = qt * BQ;
  const int last = min(row0 + BQ, a.n_q) - 1;
  const int maxpos = a.qpos[last];
  const int kbeg = split * a.split_len;
  if (kbeg > maxpos) return;
  const int kend = min(min(kbeg + a.split_len, maxpos + 1), a.n_tok);
  const int minpos = a.qpos[row0];
  const int ntiles = (kend - kbeg + BKV - 1) / BKV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = g * G + wave;
  const int l16 = lane & 15, lg = lane >> 4;
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q);
  const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + g * DH;
  const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + g * DH;
  const long kv_row = (long)a.hkv * DH;
  const float c = a.scale_log2;

  int mypos[RB];
  bf16x8_t qf[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 16 + l16;
    const bool ok = r < a.n_q;
    mypos[rb] = ok ? a.qpos[r] : -1;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qf[rb][ds] = ok ? *reinterpret_cast<const bf16x8_t*>(Q + (long)r * a.ldq + h * DH + ds * 32 + lg * 8)
                      : bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }
  float m_i[RB], l_i[RB];
  f32x4_t o[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_i[rb] = NEG_INF;
    l_i[rb] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[rb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // K and V tiles staged through registers: vector v < 1024 is K (row v/16, 8 dims at
  // 8*(v%16)), the rest V.  Keys past kend read key 0 (finite; masked out below).
  u32x4_t rg[L_PT];
#define CB_ALOAD(KT)                                                                                  \
  _Pragma("unroll") for (int i = 0; i < L_PT; ++i) {                                                 \
    const int v = tid + NT * i;                                                                      \
    if (NVEC % NT == 0 || v < NVEC) {                                                                \
      const int w = v & 1023;                                                                        \
      int key = (KT) + (w >> 4);                                                                     \
      key = key < kend ? key : 0;                                                                    \
      const bf16_t* src = (v < 1024 ? Kg : Vg) + key * kv_row + (w & 15) * 8;                        \
      rg[i] = *reinterpret_cast<const u32x4_t*>(src);                                                \
    }                                                                                                \
  }
#define CB_AWRITE(ST)                                                                                 \
  _Pragma("unroll") for (int i = 0; i < L_PT; ++i) {                                                 \
    const int v = tid + NT * i;                                                                      \
    if (NVEC % NT == 0 || v < NVEC) {                                                                \
      const int w = v & 1023;                                                                        \
      bf16_t* dst = v < 1024 ? &Ks[ST][(w >> 4) * KP + (w & 15) * 8] : &Vs[ST][(w >> 4) * VP + (w & 15) * 8]; \
      *reinterpret_cast<u32x4_t*>(dst) = rg[i];                                                      \
    }                                                                                                \
  }

  CB_ALOAD(kbeg);
  CB_AWRITE(0);
  __syncthreads();
  // V^T fragment addressing for the transpose reads: lane (group lg, j = l16) reads 8 bytes of key
  // row 4*lg + j/4 (+16 for the second half), dims 16*d + 4*(j%4); it receives V[4 keys][dim 16*d + j].
  const int vt_off = (4 * lg + (l16 >> 2)) * VP + 4 * (l16 & 3);
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    const int kt = kbeg + t * BKV;
    const bool more = t + 1 < ntiles;
    if (more) { CB_ALOAD(kt + BKV); }

    f32x4_t s[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&Ks[st][(kb * 16 + l16) * KP + ds * 32 + lg * 8]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[rb][ds], s[rb][kb], 0, 0, 0);
      }
    // s[rb][kb][r] = raw score of row (rb*16 + l16) and key kt + 16*kb + 4*lg + r
    const bool edge = (kt + BKV > kend) || (kt + BKV - 1 > minpos);
    bf16x8_t pf[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (edge) {
        const int thr = min(mypos[rb], kend - 1) - kt - 4 * lg;  // key offset 16*kb + r must be <= thr
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[rb][kb][r] = (kb * 16 + r <= thr) ? s[rb][kb][r] : NEG_INF;
      }
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mx = fmaxf(mx, fmaxf(fmaxf(s[rb][kb][0], s[rb][kb][1]), fmaxf(s[rb][kb][2], s[rb][kb][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_i[rb], mx);
      const float alpha = (m_new == m_i[rb]) ? 1.f : __builtin_amdgcn_exp2f((m_i[rb] - m_new) * c);
      const float mc = (m_new == NEG_INF) ? 0.f : m_new * c;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[rb][kb][r], c, -mc));
          s[rb][kb][r] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_i[rb] = l_i[rb] * alpha + rs;
      m_i[rb] = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int d = 0; d < 8; ++d) o[rb][d] *= alpha;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4_t w = {pack_bf16x2(s[rb][2 * ks][0], s[rb][2 * ks][1]), pack_bf16x2(s[rb][2 * ks][2], s[rb][2 * ks][3]),
                           pack_bf16x2(s[rb][2 * ks + 1][0], s[rb][2 * ks + 1][1]),
                           pack_bf16x2(s[rb][2 * ks + 1][2], s[rb][2 * ks + 1][3])};
        pf[rb][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16_t* vp = &Vs[st][ks * 32 * VP + d * 16 + vt_off];
        const u32x2_t lo = lds_read_tr16(vp);
        const u32x2_t hi = lds_read_tr16(vp + 16 * VP);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[rb][ks], o[rb][d], 0, 0, 0);
      }
    if (more) { CB_AWRITE(st ^ 1); }
    __syncthreads();
  }
#undef CB_ALOAD
#undef CB_AWRITE

  // o[rb][d][r] = O[row rb*16 + l16][d*16 + 4*lg + r]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int my_row = row0 + rb * 16 + l16;
    if (my_row >= a.n_q) continue;
    if (a.splits == 1) {
      const float inv = l_i[rb] > 0.f ? 1.f / l_i[rb] : 0.f;
      bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + (long)my_row * a.ldo + h * DH + lg * 4;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<u32x2_t*>(out + d * 16) =
            u32x2_t{pack_bf16x2(o[rb][d][0] * inv, o[rb][d][1] * inv), pack_bf16x2(o[rb][d][2] * inv, o[rb][d][3] * inv)};
    } else {
      const long idx = ((long)split * a.n_q + my_row) * a.hq + h;
      float* po = a.part_o + idx * DH + lg * 4;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<float4*>(po + d * 16) = make_float4(o[rb][d][0], o[rb][d][1], o[rb][d][2], o[rb][d][3]);
      if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + idx * 2) = make_float2(m_i[rb] * c, l_i[rb]);
    }
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

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
  const int rows = attn_rows_per_wg(a.n_q);
  dim3 grid(((a.n_q + rows - 1) / rows) * a.hkv, a.splits);
  if (rows == 32)
    hipLaunchKernelGGL((attn_bf16_kernel<G, 2>), grid, dim3(64 * G), 0, s, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<G, 1>), grid, dim3(64 * G), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int attn_rows_per_wg(int n_q) { return n_q >= 2048 ? 32 : 16; }

hipError_t attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_q <= 0) return hipSuccess;
  hipError_t e;
  switch (a.hq / a.hkv) {
    case 1: e = launch_g<1>(a, s); break;
    case 2: e = launch_g<2>(a, s); break;
    case 4: e = launch_g<4>(a, s); break;
    case 6: e = launch_g<6>(a, s); break;
    case 7: e = launch_g<7>(a, s); break;
    case 8: e = launch_g<8>(a, s); break;
    default: return hipErrorInvalidValue;
  }
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
