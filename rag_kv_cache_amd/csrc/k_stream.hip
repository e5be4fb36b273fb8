// Streaming kernels of the fusion step: embedding gather, RMSNorm, the RoPE position
// update of cached K, and the fused deviation-score + scatter of fresh K/V rows.
// All of them are HBM-bound; they use 16-byte vector accesses with consecutive lanes on
// consecutive addresses, one wavefront (64 lanes) per row where a row reduction is needed.
#include "cb_common.h"
#include "cb_kernels.h"

namespace cb {
namespace {

// ---------------------------------------------------------------- embedding gather
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tok, int n, const T* table, int vocab, int d,
                                                    float* out) {
  const int row = blockIdx.x;
  if (row >= n) return;
  const int t = tok[row];
  float* o = out + (long)row * d;
  constexpr int VE = Vec16<T>::N;
  for (int e = threadIdx.x * VE; e < d; e += blockDim.x * VE) {
    float v[VE];
    if (t >= 0 && t < vocab) {
      Vec16<T>::load(table + (long)t * d + e, v);
    } else {
#pragma unroll
      for (int i = 0; i < VE; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < VE; i += 4) *reinterpret_cast<float4*>(o + e + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  }
}

// ---------------------------------------------------------------- RMSNorm
// out[r] = h[r] / sqrt(mean(h[r]^2) + eps) * g, one wavefront per row, fp32 math.  Lane l
// owns elements 4l + 256k; the sum of squares adds them in increasing k (then a fixed
// butterfly).
template <typename TO>
__device__ __forceinline__ void store4(TO* o, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* o, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(o) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* o, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(o) = make_uint2((uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16),
                                            (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16));
}

__device__ __forceinline__ float sq4(float4 v) { return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w; }

// Sum of squares of one row (d % 4 == 0): lane l adds its 16-byte blocks k = 0, 1, ... (elements
// 4l + 256k) in increasing k, then the wave's butterfly; up to eight loads per lane in flight.
__device__ __forceinline__ float row_sumsq(const float* x, int d, int lane) {
  float ss = 0.f;
  for (int e0 = lane * 4; e0 < d; e0 += 2048) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (e0 + 256 * u < d) v[u] = *reinterpret_cast<const float4*>(x + e0 + 256 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (e0 + 256 * u < d) ss += sq4(v[u]);
  }
  return wave_sum(ss);
}

template <typename TO>
__device__ __forceinline__ void row_scale_store(const float* x, int d, const float* g, float r, TO* o, int lane) {
  for (int e = lane * 4; e < d; e += 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + e);
    const float4 gg = *reinterpret_cast<const float4*>(g + e);
    store4<TO>(o + e, v.x * r * gg.x, v.y * r * gg.y, v.z * r * gg.z, v.w * r * gg.w);
  }
}

// Rows of at most 256 U elements: the whole row in registers, every load in flight at once (the
// gains with it when GG), one read of the row.
template <typename TO, int U, bool GG>
__device__ __forceinline__ void rmsnorm_row_regs(const float* x, int d, const float* g, float eps, TO* o, int lane) {
  float4 v[U], gg[GG ? U : 1];
  const int e0 = lane * 4;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (e0 + 256 * u < d) {
      v[u] = *reinterpret_cast<const float4*>(x + e0 + 256 * u);
      if constexpr (GG) gg[u] = *reinterpret_cast<const float4*>(g + e0 + 256 * u);
    }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (e0 + 256 * u < d) ss += sq4(v[u]);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = e0 + 256 * u;
    if (e < d) {
      const float4 q = GG ? gg[GG ? u : 0] : *reinterpret_cast<const float4*>(g + e);
      store4<TO>(o + e, v[u].x * r * q.x, v[u].y * r * q.y, v[u].z * r * q.z, v[u].w * r * q.w);
    }
  }
}

// W = 0: rows up to 2048 wide; W = 1: up to 8192 (128 registers of row, the gains, L2-resident,
// loaded after the sum; a separate instantiation so that the narrow rows keep their occupancy);
// W = 2: any width, the row read twice.  The sum of squares has the same order in all three.
template <typename TO, int W>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* h, long ldh, int n, int d, const float* g,
                                                      float eps, TO* out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float* x = h + (long)row * ldh;
  TO* o = out + (long)row * d;
  if constexpr (W == 0) {
    rmsnorm_row_regs<TO, 8, true>(x, d, g, eps, o, lane);
  } else if constexpr (W == 1) {
    rmsnorm_row_regs<TO, 32, false>(x, d, g, eps, o, lane);
  } else {
    const float ss = row_sumsq(x, d, lane);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    row_scale_store<TO>(x, d, g, r, o, lane);
  }
}

// ---------------------------------------------------------------- RoPE position update
// For context row j of chunk c (offset o_c): K_f[j] = R(o_c) K_c[j] (half-split pairs
// (i, i + dh/2), cos/sin of o_c * theta_i from the fp64-built table), V_f[j] = V_c[j] when
// copy_v.  One work item = VE consecutive pairs of one head of one row: two 16-byte loads
// (first and second half), two 16-byte stores.
template <typename T>
__global__ __launch_bounds__(256) void rope_delta_kernel(const T* kc, const T* vc, T* kf, T* vf, int n_ctx,
                                                         int hkv, int dh, const int32_t* offs, int n_chunks,
                                                         const float2* table, int table_rows, int copy_v) {
  constexpr int VE = Vec16<T>::N;
  constexpr int MAXC = 256;  // chunk offsets searched in LDS (more chunks: searched in global memory)
  __shared__ int s_offs[MAXC + 1];
  const bool in_lds = n_chunks <= MAXC;
  if (in_lds)
    for (int i = threadIdx.x; i <= n_chunks; i += blockDim.x) s_offs[i] = offs[i];
  __syncthreads();
  const int half = dh >> 1;
  const int vph = half / VE;
  const int vpr = hkv * vph;
  const long total = (long)n_ctx * vpr;
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += (long)gridDim.x * blockDim.x) {
    const int row = (int)(it / vpr);
    const int rem = (int)(it - (long)row * vpr);
    const int h = rem / vph;
    const int i0 = (rem - h * vph) * VE;
    int lo = 0, hi = n_chunks - 1;  // last chunk whose offset <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((in_lds ? s_offs[mid] : offs[mid]) <= row) lo = mid; else hi = mid - 1;
    }
    int o = in_lds ? s_offs[lo] : offs[lo];
    o = o < 0 ? 0 : (o >= table_rows ? table_rows - 1 : o);  // the device offsets are not host-checked
    const long base = ((long)row * hkv + h) * dh + i0;
    float a[VE], b[VE], ya[VE], yb[VE];
    Vec16<T>::load(kc + base, a);
    Vec16<T>::load(kc + base + half, b);
    uint4 v0, v1;
    if (copy_v) {
      v0 = *reinterpret_cast<const uint4*>(vc + base);
      v1 = *reinterpret_cast<const uint4*>(vc + base + half);
    }
    const float2* cs = table + (long)o * half + i0;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const float2 t = cs[e];
      ya[e] = a[e] * t.x - b[e] * t.y;
      yb[e] = b[e] * t.x + a[e] * t.y;
    }
    Vec16<T>::store(kf + base, ya);
    Vec16<T>::store(kf + base + half, yb);
    if (copy_v) {
      *reinterpret_cast<uint4*>(vf + base) = v0;
      *reinterpret_cast<uint4*>(vf + base + half) = v1;
    }
  }
}

// The same position update for several layers in one launch: blockIdx.y = layer; every layer
// has its own cache and fused buffers (same shape, same chunk offsets).
template <typename T>
__global__ __launch_bounds__(256) void rope_delta_layers_kernel(RopeLayers L, int n_ctx, int hkv, int dh,
                                                                const int32_t* offs, int n_chunks,
                                                                const float2* table, int table_rows, int copy_v) {
  constexpr int VE = Vec16<T>::N;
  constexpr int MAXC = 256;
  __shared__ int s_offs[MAXC + 1];
  const bool in_lds = n_chunks <= MAXC;
  if (in_lds)
    for (int i = threadIdx.x; i <= n_chunks; i += blockDim.x) s_offs[i] = offs[i];
  __syncthreads();
  const int l = blockIdx.y;
  const T* kc = reinterpret_cast<const T*>(L.kc[l]);
  const T* vc = reinterpret_cast<const T*>(L.vc[l]);
  T* kf = reinterpret_cast<T*>(L.kf[l]);
  T* vf = reinterpret_cast<T*>(L.vf[l]);
  const int half = dh >> 1;
  const int vph = half / VE;
  const int vpr = hkv * vph;
  const long total = (long)n_ctx * vpr;
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += (long)gridDim.x * blockDim.x) {
    const int row = (int)(it / vpr);
    const int rem = (int)(it - (long)row * vpr);
    const int h = rem / vph;
    const int i0 = (rem - h * vph) * VE;
    int lo = 0, hi = n_chunks - 1;  // last chunk whose offset <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((in_lds ? s_offs[mid] : offs[mid]) <= row) lo = mid; else hi = mid - 1;
    }
    int o = in_lds ? s_offs[lo] : offs[lo];
    o = o < 0 ? 0 : (o >= table_rows ? table_rows - 1 : o);  // the device offsets are not host-checked
    const long base = ((long)row * hkv + h) * dh + i0;
    float a[VE], b[VE], ya[VE], yb[VE];
    Vec16<T>::load(kc + base, a);
    Vec16<T>::load(kc + base + half, b);
    uint4 v0, v1;
    if (copy_v) {
      v0 = *reinterpret_cast<const uint4*>(vc + base);
      v1 = *reinterpret_cast<const uint4*>(vc + base + half);
    }
    const float2* cs = table + (long)o * half + i0;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const float2 t = cs[e];
      ya[e] = a[e] * t.x - b[e] * t.y;
      yb[e] = b[e] * t.x + a[e] * t.y;
    }
    Vec16<T>::store(kf + base, ya);
    Vec16<T>::store(kf + base + half, yb);
    if (copy_v) {
      *reinterpret_cast<uint4*>(vf + base) = v0;
      *reinterpret_cast<uint4*>(vf + base + half) = v1;
    }
  }
}

// ---------------------------------------------------------------- fetch from pinned host memory
// fetch_kv in one pass: the kernel reads one layer's cached rows of every chunk straight from
// pinned host memory (over PCIe), rotates K by R(o_c) and copies V into the fused buffers in
// device memory.  A few workgroups of 1024 threads, each thread with the host loads of FU items
// in flight: the link, not the number of workgroups, bounds it, and the compute kernels keep
// the other CUs.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4 v, float* o);
template <>
__device__ __forceinline__ void unpack16<float>(const uint4 v, float* o) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4 v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T, int FU>
__global__ __launch_bounds__(1024) void fetch_rope_kernel(FetchChunks F, T* kf, T* vf, int hkv, int dh,
                                                         const float2* table, int table_rows) {
  constexpr int VE = Vec16<T>::N;
  const int half = dh >> 1;
  const int vph = half / VE;
  const int vpr = hkv * vph;
  const int r0 = F.offs[0];
  const long total = (long)(F.offs[F.n] - r0) * vpr;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long it0 = (long)blockIdx.x * blockDim.x + threadIdx.x; it0 < total; it0 += stride * FU) {
    uint4 k0[FU], k1[FU], v0[FU], v1[FU];
    long dst[FU];
    int off[FU], i0s[FU];
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      const long it = it0 + u * stride;
      dst[u] = -1;
      if (it >= total) continue;
      const int row = r0 + (int)(it / vpr);
      const int rem = (int)(it - (long)(row - r0) * vpr);
      const int h = rem / vph;
      const int i0 = (rem - h * vph) * VE;
      int lo = 0, hi = F.n - 1;  // last chunk whose first row <= row
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (F.offs[mid] <= row) lo = mid; else hi = mid - 1;
      }
      const long src = ((long)(row - F.offs[lo]) * hkv + h) * dh + i0;
      const T* hk = reinterpret_cast<const T*>(F.hk[lo]) + src;
      const T* hv = reinterpret_cast<const T*>(F.hv[lo]) + src;
      k0[u] = *reinterpret_cast<const uint4*>(hk);
      k1[u] = *reinterpret_cast<const uint4*>(hk + half);
      v0[u] = *reinterpret_cast<const uint4*>(hv);
      v1[u] = *reinterpret_cast<const uint4*>(hv + half);
      int o = F.offs[lo];
      off[u] = o < 0 ? 0 : (o >= table_rows ? table_rows - 1 : o);
      i0s[u] = i0;
      dst[u] = ((long)row * hkv + h) * dh + i0;
    }
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      if (dst[u] < 0) continue;
      float a[VE], b[VE], ya[VE], yb[VE];
      unpack16<T>(k0[u], a);
      unpack16<T>(k1[u], b);
      const float2* cs = table + (long)off[u] * half + i0s[u];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float2 t = cs[e];
        ya[e] = a[e] * t.x - b[e] * t.y;
        yb[e] = b[e] * t.x + a[e] * t.y;
      }
      Vec16<T>::store(kf + dst[u], ya);
      Vec16<T>::store(kf + dst[u] + half, yb);
      *reinterpret_cast<uint4*>(vf + dst[u]) = v0[u];
      *reinterpret_cast<uint4*>(vf + dst[u] + half) = v1[u];
    }
  }
}

// ---------------------------------------------------------------- deviation + scatter
// One wavefront per recomputed row i (position j = sel[i]): for context rows (i < n_cand)
// dev[i] = sum over the row's K and V elements of (fresh - fused)^2, read before the
// fused row is overwritten; then fused[j] <- fresh[i].  fresh row layout: K heads then
// V heads (row_elems each).  LPR lanes per row (the row's 16-byte pieces, at most 64: a
// wavefront holds 64 / LPR rows, so narrow rows still use every lane), each piece's loads issued
// before any use.  Per-lane sequential sums then a fixed butterfly over the row's lanes: the
// result does not depend on scheduling.
// When the layer keeps every recomputed row (copy_sel set), the kept set is sel itself:
// copy_sel[i] = sel[i], copy_local[i] = i.  cosine != 0 scores 1 - <fresh, fused> /
// (|fresh| |fused|) over the row's K and V instead of the squared distance (0 when both rows
// are zero, 1 when only one is).
template <typename T, int LPR>
__global__ __launch_bounds__(256) void dev_scatter_kernel(const T* fresh, long ld_fresh, T* fk, T* fv,
                                                          const int32_t* sel, int n_sel, int n_cand, int n_tok,
                                                          int row_elems, float* dev, int32_t* copy_sel,
                                                          int32_t* copy_local, int cosine) {
  constexpr int VE = Vec16<T>::N;
  constexpr int RPW = 64 / LPR;  // rows per wavefront, LPR lanes each
  const int lane = threadIdx.x & 63, l = lane % LPR;
  const int i = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const bool valid = i < n_sel;
  const int j = valid ? sel[i] : -1;
  if (valid && copy_sel && l == 0) {
    copy_sel[i] = j;
    copy_local[i] = i;
  }
  const bool score = dev != nullptr && valid && i < n_cand;
  const bool ok = valid && j >= 0 && j < n_tok;
  float acc = 0.f, na = 0.f, nb = 0.f;
  if (ok) {
    const T* fr = fresh + (long)i * ld_fresh;
    T* dk = fk + (long)j * row_elems;
    T* dv = fv + (long)j * row_elems;
    for (int e = l * VE; e < row_elems; e += LPR * VE) {
      // every load of the piece first (fresh K and V, and the fused rows they replace)
      const uint4 nk = *reinterpret_cast<const uint4*>(fr + e);
      const uint4 nv = *reinterpret_cast<const uint4*>(fr + row_elems + e);
      uint4 ok4 = make_uint4(0, 0, 0, 0), ov4 = make_uint4(0, 0, 0, 0);
      if (score) {
        ok4 = *reinterpret_cast<const uint4*>(dk + e);
        ov4 = *reinterpret_cast<const uint4*>(dv + e);
      }
      if (score) {
        float a[VE], b[VE];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint4 x = half ? nv : nk, y = half ? ov4 : ok4;
          Vec16<T>::load(reinterpret_cast<const T*>(&x), a);
          Vec16<T>::load(reinterpret_cast<const T*>(&y), b);
          if (cosine) {
#pragma unroll
            for (int q = 0; q < VE; ++q) { acc += a[q] * b[q]; na += a[q] * a[q]; nb += b[q] * b[q]; }
          } else {
#pragma unroll
            for (int q = 0; q < VE; ++q) { const float t = a[q] - b[q]; acc += t * t; }
          }
        }
      }
      *reinterpret_cast<uint4*>(dk + e) = nk;
      *reinterpret_cast<uint4*>(dv + e) = nv;
    }
  }
  if (dev != nullptr) {  // uniform: every lane takes part in the row sums
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) {
      acc += __shfl_xor(acc, o, 64);
      if (cosine) {
        na += __shfl_xor(na, o, 64);
        nb += __shfl_xor(nb, o, 64);
      }
    }
    if (score && l == 0) {
      if (!ok) acc = __builtin_nanf("");
      else if (cosine) acc = (na == 0.f || nb == 0.f) ? (na == nb ? 0.f : 1.f) : 1.0f - acc / (sqrtf(na) * sqrtf(nb));
      dev[i] = acc;
    }
  }
}

}  // namespace

hipError_t embed(const int32_t* tok, int n, const void* table, int vocab, int d, int bf16, float* out,
                 hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(n), dim3(256), 0, s, tok, n, (const bf16_t*)table, vocab, d, out);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(n), dim3(256), 0, s, tok, n, (const float*)table, vocab, d, out);
  return hipGetLastError();
}

hipError_t rmsnorm(const float* h, long ldh, int n, int d, const float* g, float eps, void* out, int bf16,
                   hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((n + 3) / 4);
  auto go = [&](auto kb, auto kf) {
    if (bf16) hipLaunchKernelGGL(kb, grid, dim3(256), 0, s, h, ldh, n, d, g, eps, (bf16_t*)out);
    else hipLaunchKernelGGL(kf, grid, dim3(256), 0, s, h, ldh, n, d, g, eps, (float*)out);
  };
  if (d <= 2048) go(rmsnorm_kernel<bf16_t, 0>, rmsnorm_kernel<float, 0>);
  else if (d <= 8192) go(rmsnorm_kernel<bf16_t, 1>, rmsnorm_kernel<float, 1>);
  else go(rmsnorm_kernel<bf16_t, 2>, rmsnorm_kernel<float, 2>);
  return hipGetLastError();
}

hipError_t rope_delta(const void* kc, const void* vc, void* kf, void* vf, int n_ctx, int hkv, int dh,
                      const int32_t* offs, int n_chunks, const float2* table, int table_rows, int bf16,
                      hipStream_t s) {
  if (n_ctx <= 0) return hipSuccess;
  const int ve = bf16 ? 8 : 4;
  const long items = (long)n_ctx * hkv * (dh / 2 / ve);
  long blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const int copy_v = vc != vf;
  if (bf16)
    hipLaunchKernelGGL(rope_delta_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16_t*)kc,
                       (const bf16_t*)vc, (bf16_t*)kf, (bf16_t*)vf, n_ctx, hkv, dh, offs, n_chunks, table, table_rows, copy_v);
  else
    hipLaunchKernelGGL(rope_delta_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)kc,
                       (const float*)vc, (float*)kf, (float*)vf, n_ctx, hkv, dh, offs, n_chunks, table, table_rows, copy_v);
  return hipGetLastError();
}

hipError_t rope_delta_layers(const RopeLayers& L, int n_layers, int n_ctx, int hkv, int dh, const int32_t* offs,
                             int n_chunks, const float2* table, int table_rows, int copy_v, int bf16, hipStream_t s) {
  if (n_ctx <= 0 || n_layers <= 0) return hipSuccess;
  if (n_layers > kRopeMaxLayers) return hipErrorInvalidValue;
  const int ve = bf16 ? 8 : 4;
  const long items = (long)n_ctx * hkv * (dh / 2 / ve);
  long blocks = (items + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid((unsigned)blocks, (unsigned)n_layers);
  if (bf16)
    hipLaunchKernelGGL(rope_delta_layers_kernel<bf16_t>, grid, dim3(256), 0, s, L, n_ctx, hkv, dh, offs, n_chunks,
                       table, table_rows, copy_v);
  else
    hipLaunchKernelGGL(rope_delta_layers_kernel<float>, grid, dim3(256), 0, s, L, n_ctx, hkv, dh, offs, n_chunks,
                       table, table_rows, copy_v);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fetch(const FetchChunks& F, T* kf, T* vf, int hkv, int dh, const float2* table, int table_rows,
                        const FetchLaunch& fl, hipStream_t s) {
  const dim3 grid(fl.blocks), block(fl.threads);
  switch (fl.unroll) {
    case 1: hipLaunchKernelGGL((fetch_rope_kernel<T, 1>), grid, block, 0, s, F, kf, vf, hkv, dh, table, table_rows); break;
    case 2: hipLaunchKernelGGL((fetch_rope_kernel<T, 2>), grid, block, 0, s, F, kf, vf, hkv, dh, table, table_rows); break;
    case 4: hipLaunchKernelGGL((fetch_rope_kernel<T, 4>), grid, block, 0, s, F, kf, vf, hkv, dh, table, table_rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t fetch_rope(const FetchChunks& F, void* kf, void* vf, int hkv, int dh, const float2* table, int table_rows,
                      int bf16, const FetchLaunch& fl, hipStream_t s) {
  if (F.n <= 0 || F.offs[F.n] <= F.offs[0]) return hipSuccess;
  if (F.n > kFetchMaxChunks || fl.blocks < 1 || fl.threads < 64 || fl.threads > 1024 || fl.threads % 64)
    return hipErrorInvalidValue;
  if (bf16) return launch_fetch(F, (bf16_t*)kf, (bf16_t*)vf, hkv, dh, table, table_rows, fl, s);
  return launch_fetch(F, (float*)kf, (float*)vf, hkv, dh, table, table_rows, fl, s);
}

hipError_t dev_scatter(const void* fresh, long ld_fresh, void* fk, void* fv, const int32_t* sel, int n_sel,
                       int n_cand, int n_tok, int row_elems, float* dev, int32_t* copy_sel, int32_t* copy_local,
                       int cosine, int bf16, hipStream_t s) {
  if (n_sel <= 0) return hipSuccess;
  // lanes per row: the row's 16-byte pieces, at most 64 (wider rows loop), at least 16
  const int pieces = row_elems / (bf16 ? 8 : 4);
  const int lpr = pieces >= 64 ? 64 : (pieces >= 32 ? 32 : 16);
  if (row_elems % (bf16 ? 8 : 4) != 0) return hipErrorInvalidValue;
  const int rows_per_wg = 4 * (64 / lpr);
  dim3 grid((n_sel + rows_per_wg - 1) / rows_per_wg);
#define CB_DEV_SCATTER(T, LPR)                                                                                 \
  hipLaunchKernelGGL((dev_scatter_kernel<T, LPR>), grid, dim3(256), 0, s, (const T*)fresh, ld_fresh, (T*)fk, \
                     (T*)fv, sel, n_sel, n_cand, n_tok, row_elems, dev, copy_sel, copy_local, cosine)
  if (bf16) {
    if (lpr == 64) CB_DEV_SCATTER(bf16_t, 64);
    else if (lpr == 32) CB_DEV_SCATTER(bf16_t, 32);
    else CB_DEV_SCATTER(bf16_t, 16);
  } else {
    if (lpr == 64) CB_DEV_SCATTER(float, 64);
    else if (lpr == 32) CB_DEV_SCATTER(float, 32);
    else CB_DEV_SCATTER(float, 16);
  }
#undef CB_DEV_SCATTER
  return hipGetLastError();
}

}  // namespace cb
