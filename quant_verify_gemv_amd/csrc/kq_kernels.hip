// kq_kernels.hip -- HIP kernels for the Q4_K batched verify step on gfx950.
//
// Three kernels:
//  * kq_stage_kernel: fp32 activation rows -> the MFMA operand format: per
//    row and 1,024-column quad a power-of-two scale, then each scaled value
//    split into an fp16 pair hi + lo (|x - hi - lo| <= 2^-22 |x| in range),
//    laid out in the lane order the weight unpack produces, plus the scaled
//    32-column sub-block sums the min term needs.
//  * kq_gemv_kernel<NT>: streams each 144-byte super-block once for all rows,
//    unpacks 4-bit quants times their 6-bit sub-block scale into exact fp16
//    (q * sc <= 945), and contracts them with the staged rows on
//    v_mfma_f32_16x16x32_f16 (16 rows x 16 outputs x 32 columns). The block
//    scale d and the 1/2^e row scale are applied in fp32; the min term
//    -dmin * m_j * sum(x over sub-block j) runs as three more MFMAs per quad.
//    Split-K partials are combined in fixed split order by the last
//    workgroup to arrive; in verify mode each workgroup column also takes the
//    row argmax (ties -> lowest index) and the last column to finish applies
//    the greedy accept rule.
//  * kq_fill_kernel: zeroes control words.
//
// The format (muser-book ch. 8 "The DFlash draft", section 8.2) and the
// accept rule (ch. 33 "Speculation: the local win and the distributed
// verdict", section 33.2, temperature-0 limit) are described in kq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_internal.h"

namespace kq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2v as_h2(unsigned u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ unsigned as_u(half2v h) { return __builtin_bit_cast(unsigned, h); }
__device__ __forceinline__ float h2f_lo(unsigned u) { return (float)as_h2(u)[0]; }
__device__ __forceinline__ float h2f_hi(unsigned u) { return (float)as_h2(u)[1]; }

__device__ __forceinline__ half8 make_h8(unsigned a, unsigned b, unsigned c, unsigned d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ u32x4 ld16_stream(const uint8_t *p) { return *(const u32x4 *)p; }

// Cross-workgroup hand-off without device-scope fences. Values another
// workgroup will read are written with agent-scope relaxed atomic stores
// (write-through to the device coherence point) and read back with
// agent-scope relaxed atomic loads (never served from a stale cache); the
// writer waits for its stores to complete (vmcnt(0)) before the arrival
// counter is incremented. This is the device-scope release/acquire
// sequence minus the L2 write-back/invalidate that only ordinary cached
// stores need, which would otherwise cost every workgroup an L2 flush.
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's global stores have completed, then barrier
__device__ __forceinline__ void stores_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
}
__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *(const u32x4 *)p; }

// Ordered 64-bit argmax key: larger value wins, equal values -> lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, unsigned n) {
  v = v + 0.0f;  // -0 -> +0 so that the two zeros tie
  unsigned u = __float_as_uint(v);
  unsigned ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - n);
}

// ---------------------------------------------------------------------------
// Staging. One workgroup per quad, thread t handles row m = t/16 and the 64
// columns c = t%16 of the quad (block bq = c/4 within the quad, 64-weight
// group grp = c%4 of that block).
__global__ __launch_bounds__(256) void kq_stage_kernel(const float *__restrict__ x, int m_rows,
                                                       int64_t k, uint8_t *__restrict__ staged,
                                                       unsigned *__restrict__ zero_words,
                                                       int64_t n_zero_words) {
  const int t = threadIdx.x;
  const int m = t >> 4;
  const int c = t & 15;
  const int bq = c >> 2, grp = c & 3;
  const int64_t q = blockIdx.x;
  const int64_t k0 = q * kQuadK + 64 * c;
  const bool valid = k0 < k;
  const bool active = m < m_rows;  // rows >= m_rows are staged as zeros

  if (zero_words && q == 0) {
    for (int64_t i = t; i < n_zero_words; i += 256) zero_words[i] = 0u;
  }

  float v[64];
  float amax = 0.0f;
  if (active && valid) {
    const f32x4 *src = (const f32x4 *)(x + (int64_t)m * k + k0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f32x4 f = src[i];
      v[4 * i + 0] = f[0]; v[4 * i + 1] = f[1]; v[4 * i + 2] = f[2]; v[4 * i + 3] = f[3];
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = 0.0f;
  }
  // max over the 16 threads of row m (16 consecutive lanes of one wave)
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));

  // scale 2^e puts the quad's largest magnitude in [2^9, 2^10): scaled values
  // and their 32-term sums stay inside fp16 range.
  int e = 0;
  if (amax > 0.0f) {
    int E;
    (void)frexpf(amax, &E);
    e = 10 - E;
    e = e > 100 ? 100 : e;
  }
  // rows >= m_rows are staged as zeros with scale 1: the main kernel then
  // runs every row unpredicated and simply does not store rows >= m.
  uint8_t *qbase = staged + q * kQuadBytes;
  if (c == 0) *(float *)(qbase + kXiOffset + 4 * m) = ldexpf(1.0f, -e);

  const int lane_l = m + 16 * grp;   // lane index of this row/group in XA
  const int lane_s = m + 16 * bq;    // lane index of this row/block in XS
  if (!valid) {
    *(unsigned *)(qbase + kXsOffset + 0 * 1024 + lane_s * 16 + grp * 4) = 0u;
    *(unsigned *)(qbase + kXsOffset + 1 * 1024 + lane_s * 16 + grp * 4) = 0u;
    return;
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = ldexpf(v[i], e);

  // sub-block sums (sub-block 2*grp = first 32 columns, 2*grp+1 = next 32)
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s0 += v[i];
#pragma unroll
  for (int i = 32; i < 64; ++i) s1 += v[i];
  {
    _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
    _Float16 l0 = (_Float16)(s0 - (float)h0), l1 = (_Float16)(s1 - (float)h1);
    half2v hh = {h0, h1}, ll = {l0, l1};
    *(unsigned *)(qbase + kXsOffset + 0 * 1024 + lane_s * 16 + grp * 4) = as_u(hh);
    *(unsigned *)(qbase + kXsOffset + 1 * 1024 + lane_s * 16 + grp * 4) = as_u(ll);
  }

  // XA: k-step s takes 8 columns of the group in the order the weight unpack
  // produces them: bytes {0,2,1,3} of two consecutive quant dwords.
  const int perm[4] = {0, 2, 1, 3};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int sp = s & 3, half = s >> 2;
    unsigned hw[4], lw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i0 = 2 * p, i1 = 2 * p + 1;
      const float x0 = v[32 * half + 8 * sp + 4 * (i0 >> 2) + perm[i0 & 3]];
      const float x1 = v[32 * half + 8 * sp + 4 * (i1 >> 2) + perm[i1 & 3]];
      _Float16 a0 = (_Float16)x0, a1 = (_Float16)x1;
      _Float16 b0 = (_Float16)(x0 - (float)a0), b1 = (_Float16)(x1 - (float)a1);
      half2v ha = {a0, a1}, hb = {b0, b1};
      hw[p] = as_u(ha);
      lw[p] = as_u(hb);
    }
    uint8_t *dst = qbase + (int64_t)bq * kXaBlockBytes + (int64_t)(s * 2) * 1024 + lane_l * 16;
    *(u32x4 *)dst = u32x4{hw[0], hw[1], hw[2], hw[3]};
    *(u32x4 *)(dst + 1024) = u32x4{lw[0], lw[1], lw[2], lw[3]};
  }
}

// ---------------------------------------------------------------------------

__global__ void kq_fill_kernel(unsigned *p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Main kernel. Workgroup (blockIdx.x, blockIdx.y) covers rows
// [64*NT*blockIdx.x, +64*NT) -- wave w owns tiles 4*NT*blockIdx.x... -- and
// quads [qps*blockIdx.y, +qps). Lane l of a wave: ln = l%16 is both the
// output row within a tile (B operand / C column) and the activation row m
// of the A operand; kg = l/16 selects the 64-weight group of each block the
// lane unpacks (sub-blocks 2kg, 2kg+1) and the C rows 4kg..4kg+3.

struct WTile {
  u32x4 hdr, q0, q1;
};

template <int NT>
__global__ __launch_bounds__(256) void kq_gemv_kernel(GemvLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kXaBlockBytes];
  __shared__ unsigned long long s_keys[kMaxRows];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kg = lane >> 4;
  const int ln = lane & 15;
  const int M = a.m;

  const int64_t N = a.n;
  const int64_t KB = a.k / kQK;
  const int tile0 = (blockIdx.x * kWaves + wave) * NT;
  int64_t rows[NT];
  const uint8_t *rowp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    rows[t] = (int64_t)(tile0 + t) * 16 + ln;
    const int64_t r = rows[t] < N ? rows[t] : N - 1;
    rowp[t] = a.w + r * a.row_bytes;
  }

  const int q_begin = blockIdx.y * a.g.qps;
  const int q_end = min(a.g.quads, q_begin + a.g.qps);
  const int64_t b_begin = (int64_t)q_begin * 4;
  const int64_t b_last = min(KB, (int64_t)q_end * 4) - 1;  // last block of this split

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline. The weights of a wave's NT tiles rotate through four
  // register sets (the quad loop is unrolled four times, one step per block)
  // so that the loads of block b+3 are in flight while block b computes; the
  // activations of block b+1 are loaded during block b and written to the
  // other LDS buffer at its end. Every load is unconditional (indices are
  // clamped to the split's last block) so that outstanding loads are counted
  // statically and waits cover only the data about to be used.
  auto clampb = [&](int64_t b) -> int64_t { return b < b_last ? b : b_last; };
  auto load_w = [&](WTile (&w)[NT], int64_t b) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t *p = rowp[t] + b * kBlockBytes;
      w[t].hdr = ld16_stream(p);
      w[t].q0 = ld16_stream(p + 16 + 32 * kg);
      w[t].q1 = ld16_stream(p + 32 + 32 * kg);
    }
  };
  auto x_src = [&](int64_t b) -> const uint8_t * {
    return a.staged + (b >> 2) * kQuadBytes + (b & 3) * kXaBlockBytes;
  };
  WTile w0[NT], w1[NT], w2[NT], w3[NT];
  load_w(w0, b_begin);
  load_w(w1, clampb(b_begin + 1));
  load_w(w2, clampb(b_begin + 2));
  {
    const uint8_t *src = x_src(b_begin);
    u32x4 xr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xr[j] = ld16(src + (tid + 256 * j) * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4 *)(&s_x[0][(tid + 256 * j) * 16]) = xr[j];
  }
  __syncthreads();

  for (int q = q_begin; q < q_end; ++q) {
    const uint8_t *qb = a.staged + (int64_t)q * kQuadBytes;
    const u32x4 xs_hi = ld16(qb + kXsOffset + lane * 16);
    const u32x4 xs_lo = ld16(qb + kXsOffset + 1024 + lane * 16);
    const f32x4 xinv = *(const f32x4 *)(qb + kXiOffset + 16 * kg);
    const int64_t qb0 = (int64_t)q * 4;
    const int nblk = (int)(min((int64_t)4, b_last + 1 - qb0));
    f32x4 G[NT];
    u32x4 hmin[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      G[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      hmin[t] = u32x4{0u, 0u, 0u, 0u};
    }

    // one block: prefetch block b+3 into `pf` and activations of b+1, then
    // contract the weights in `cur` with the activations in LDS buffer bq&1.
    auto step = [&](WTile (&cur)[NT], WTile (&pf)[NT], const int bq) {
      const int64_t b = qb0 + bq;
      u32x4 xr[4];
      {
        const uint8_t *src = x_src(clampb(b + 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[j] = ld16(src + (tid + 256 * j) * 16);
      }
      load_w(pf, clampb(b + 3));
      __builtin_amdgcn_sched_barrier(0);
      if (bq < nblk) {
        unsigned slo[NT], nlo[NT], shi[NT], nhi[NT];
        float dsc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const u32x4 h = cur[t].hdr;
          hmin[t] = bq == kg ? h : hmin[t];
          dsc[t] = h2f_lo(h.x);
          const unsigned sc03 = h.y & 0x3F3F3F3Fu;
          const unsigned sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
          const unsigned sel = (kg < 2 ? sc03 : sc47) >> ((kg & 1) * 16);
          const float s0 = (float)(sel & 0xFFu);         // sc[2kg]   (low nibbles)
          const float s1 = (float)((sel >> 8) & 0xFFu);  // sc[2kg+1] (high nibbles)
          half2v a0 = {(_Float16)s0, (_Float16)s0};
          half2v a1 = {(_Float16)(-1024.0f * s0), (_Float16)(-1024.0f * s0)};
          half2v a2 = {(_Float16)(0.0625f * s1), (_Float16)(0.0625f * s1)};
          half2v a3 = {(_Float16)(-64.0f * s1), (_Float16)(-64.0f * s1)};
          slo[t] = as_u(a0); nlo[t] = as_u(a1); shi[t] = as_u(a2); nhi[t] = as_u(a3);
        }
        f32x4 chi[NT], clo[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          chi[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          clo[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const uint8_t *xb = s_x[bq & 1];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const half8 ahi = *(const half8 *)(xb + (s * 2 + 0) * 1024 + lane * 16);
          const half8 alo = *(const half8 *)(xb + (s * 2 + 1) * 1024 + lane * 16);
          const int sp = s & 3;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const u32x4 q0 = cur[t].q0, q1 = cur[t].q1;
            const unsigned da = sp == 0 ? q0.x : sp == 1 ? q0.z : sp == 2 ? q1.x : q1.z;
            const unsigned db = sp == 0 ? q0.y : sp == 1 ? q0.w : sp == 2 ? q1.y : q1.w;
            const unsigned mask = s < 4 ? 0x000F000Fu : 0x00F000F0u;
            const half2v sc = as_h2(s < 4 ? slo[t] : shi[t]);
            const half2v nb = as_h2(s < 4 ? nlo[t] : nhi[t]);
            const unsigned u0 = (da & mask) | 0x64006400u;
            const unsigned u1 = ((da >> 8) & mask) | 0x64006400u;
            const unsigned u2 = (db & mask) | 0x64006400u;
            const unsigned u3 = ((db >> 8) & mask) | 0x64006400u;
            const half2v v0 = __builtin_elementwise_fma(as_h2(u0), sc, nb);
            const half2v v1 = __builtin_elementwise_fma(as_h2(u1), sc, nb);
            const half2v v2 = __builtin_elementwise_fma(as_h2(u2), sc, nb);
            const half2v v3 = __builtin_elementwise_fma(as_h2(u3), sc, nb);
            const half8 bw = make_h8(as_u(v0), as_u(v1), as_u(v2), as_u(v3));
            chi[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bw, chi[t], 0, 0, 0);
            clo[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bw, clo[t], 0, 0, 0);
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int r = 0; r < 4; ++r) G[t][r] += dsc[t] * (chi[t][r] + clo[t][r]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) *(u32x4 *)(&s_x[(bq & 1) ^ 1][(tid + 256 * j) * 16]) = xr[j];
      __syncthreads();
    };
    step(w0, w3, 0);
    step(w1, w0, 1);
    step(w2, w1, 2);
    step(w3, w2, 3);

    // end of the quad: min term (three MFMAs) and the row scale 2^-e
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 h = hmin[t];
      const bool ok = kg < nblk;
      const float dmin = h2f_hi(h.x);
      const unsigned m03 = h.z & 0x3F3F3F3Fu;
      const unsigned m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
      unsigned bh[4], bl[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const unsigned src = p < 2 ? m03 : m47;
        const int sh = (p & 1) * 16;
        const float v0 = ok ? dmin * (float)((src >> sh) & 0xFFu) : 0.0f;
        const float v1 = ok ? dmin * (float)((src >> (sh + 8)) & 0xFFu) : 0.0f;
        const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
        const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
        half2v hh = {h0, h1}, ll = {l0, l1};
        bh[p] = as_u(hh);
        bl[p] = as_u(ll);
      }
      const half8 b2h = make_h8(bh[0], bh[1], bh[2], bh[3]);
      const half8 b2l = make_h8(bl[0], bl[1], bl[2], bl[3]);
      const half8 a2h = __builtin_bit_cast(half8, xs_hi);
      const half8 a2l = __builtin_bit_cast(half8, xs_lo);
      f32x4 c2 = {0.f, 0.f, 0.f, 0.f};
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2h, b2h, c2, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2l, b2h, c2, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2h, b2l, c2, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] += xinv[r] * (G[t][r] - c2[r]);
    }
  }

  // ---------------------------------------------------------------- epilogue
  const int splits = a.g.splits;
  const int wg = blockIdx.x;
  const int rows_wg = 64 * NT;
  const int64_t row0 = (int64_t)wg * rows_wg;

  if (tid < kMaxRows) s_keys[tid] = 0ull;

  if (splits == 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (rows[t] < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * kg + r;
          if (m < M && a.logits) a.logits[(int64_t)m * N + rows[t]] = acc[t][r];
        }
      }
    }
    if (a.verify) {
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kg + r;
        if (m < M) {
          unsigned long long best = 0ull;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (rows[t] < N) {
              const unsigned long long key = argmax_key(acc[t][r], (unsigned)rows[t]);
              best = key > best ? key : best;
            }
          if (best) atomicMax(&s_keys[m], best);
        }
      }
    }
  } else {
    // write this split's partial sums, then the last arriving split sums all
    // splits in split order.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (rows[t] < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * kg + r;
          if (m < M) st_dev(&a.partials[((int64_t)blockIdx.y * kMaxRows + m) * N + rows[t]], acc[t][r]);
        }
      }
    }
    stores_done_barrier();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(&a.tile_cnt[wg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == (unsigned)(splits - 1);
      if (last) __hip_atomic_store(&a.tile_cnt[wg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = last;
    }
    __syncthreads();
    if (!s_flag) return;
    const int64_t nrows = min((int64_t)rows_wg, N - row0);
    for (int64_t e = tid; e < (int64_t)M * nrows; e += kThreads) {
      const int m = (int)(e / nrows);
      const int64_t n = row0 + e % nrows;
      float v = 0.0f;
      for (int sp = 0; sp < splits; ++sp) {
        const float pv = ld_dev(&a.partials[((int64_t)sp * kMaxRows + m) * N + n]);
        v = sp == 0 ? pv : v + pv;
      }
      if (a.logits) a.logits[(int64_t)m * N + n] = v;
      if (a.verify) atomicMax(&s_keys[m], argmax_key(v, (unsigned)n));
    }
  }

  if (!a.verify) return;
  __syncthreads();
  if (tid < kMaxRows) st_dev(&a.wg_keys[(int64_t)wg * kMaxRows + tid], s_keys[tid]);
  stores_done_barrier();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag = old == (unsigned)(a.g.n_wg - 1);
  }
  __syncthreads();
  if (!s_flag) return;
  if (tid < kMaxRows) s_keys[tid] = 0ull;
  __syncthreads();
  {
    const int m = tid & 15;
    if (m < M) {
      unsigned long long best = 0ull;
      for (int w = tid >> 4; w < a.g.n_wg; w += kThreads / 16) {
        const unsigned long long key = ld_dev(&a.wg_keys[(int64_t)w * kMaxRows + m]);
        best = key > best ? key : best;
      }
      atomicMax(&s_keys[m], best);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int am[kMaxRows];
    for (int m = 0; m < M; ++m) {
      am[m] = (int)(0xFFFFFFFFu - (unsigned)(s_keys[m] & 0xFFFFFFFFull));
      a.argmax_out[m] = am[m];
    }
    int i = 0;
    while (i < a.k_draft && a.draft[i] == am[i]) ++i;
    a.accept_out[0] = i;
    a.accept_out[1] = am[i];
    __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------

int launch_stage(const float *x, int m, int64_t k, uint8_t *staged, unsigned *zero_words,
                 int64_t n_zero_words, void *stream) {
  const int64_t quads = (k + kQuadK - 1) / kQuadK;
  hipLaunchKernelGGL(kq_stage_kernel, dim3((unsigned)quads), dim3(256), 0, (hipStream_t)stream, x, m,
                     k, staged, zero_words, n_zero_words);
  return (int)hipGetLastError();
}

int launch_fill(unsigned *p, int64_t n_words, void *stream) {
  int64_t blocks = (n_words + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(kq_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p,
                     n_words);
  return (int)hipGetLastError();
}

int launch_gemv(const GemvLaunch &a, void *stream) {
  dim3 grid((unsigned)a.g.n_wg, (unsigned)a.g.splits);
  switch (a.g.nt) {
    case 1:
      hipLaunchKernelGGL(kq_gemv_kernel<1>, grid, dim3(kThreads), 0, (hipStream_t)stream, a);
      break;
    case 2:
      hipLaunchKernelGGL(kq_gemv_kernel<2>, grid, dim3(kThreads), 0, (hipStream_t)stream, a);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace kq
