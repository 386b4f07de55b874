// kq_kernels.hip -- HIP kernels for the Q4_K batched verify step on gfx950.
//
//  * kq_stage_kernel: fp32 activation rows -> the MFMA operand format: per
//    row and 1,024-column quad a power-of-two scale, then each scaled value
//    split into an fp16 pair hi + lo (|x - hi - lo| <= 2^-22 |x| in range),
//    laid out in the lane order the weight unpack produces, plus the scaled
//    32-column sub-block sums the min term needs.
//  * kq_gemv_kernel: each wave owns 16 output rows; it streams their 144-byte
//    super-blocks once for all activation rows, unpacks the 4-bit quants
//    times their 6-bit sub-block scale into exact fp16 (q * sc <= 945) and
//    contracts them with the staged rows on v_mfma_f32_16x16x32_f16 (16
//    activation rows x 16 outputs x 32 columns). The block scale d and the
//    row scale 2^-e are applied in fp32; the min term -dmin * m_j * (sum of
//    x over sub-block j) runs as three more MFMAs per quad. A launch may
//    cover several matrices that share the activations. Split-K partials are
//    combined in fixed split order by the last workgroup to arrive; in verify
//    mode every workgroup column also takes the row argmax (ties -> lowest
//    index) and the last column to finish applies the greedy accept rule.
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

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *(const u32x4 *)p; }

// A value the compiler must keep in a VGPR: lets (x & mask) | magic become
// one v_and_or_b32 (a VOP3 instruction may read one scalar operand only).
__device__ __forceinline__ unsigned in_vgpr(unsigned c) {
  unsigned v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(c));
  return v;
}

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

// Ordered 64-bit argmax key: larger value wins, equal values -> lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, unsigned n) {
  v = v + 0.0f;  // -0 -> +0 so that the two zeros tie
  unsigned u = __float_as_uint(v);
  unsigned ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - n);
}

// ---------------------------------------------------------------------------
// Lane order of the weights. Lane l of a wave: ln = l%16 is the output row
// within the 16-row tile (B operand / C column) and also the activation row
// m of the A operand; kg = l/16 selects the bytes the lane unpacks from each
// super-block: q0 = quant bytes [16kg, 16kg+16) and q1 = quant bytes
// [64+16kg, 80+16kg) (so the four lanes of a row read 64 contiguous bytes per
// load). In k-step s (0..7) the lane contributes the 8 nibbles of dwords
// 2(s&1), 2(s&1)+1 of q0 (s < 4) or q1 (s >= 4), low nibbles if (s&2) == 0,
// in the byte order {0,2,1,3,4,6,5,7} that the unpack produces. The staging
// kernel writes the activations in exactly this order.
__device__ __forceinline__ constexpr int lane_weight_index(int kg, int s, int i) {
  // byte order {0,2,1,3,4,6,5,7} within the 8 bytes of a k-step
  const int byte = (s < 4 ? 16 * kg : 64 + 16 * kg) + 8 * (s & 1) + (i & 4) + ((i & 1) << 1) + ((i >> 1) & 1);
  const int g = byte >> 5, l = byte & 31;
  return 64 * g + ((s & 2) ? 32 : 0) + l;
}

// ---------------------------------------------------------------------------
// Staging. One workgroup per quad; thread t handles row m = t/16 and the 64
// columns c = t%16 of the quad: block bq = c/4 of the quad, weight group
// grp = c%4 of that block (weights 64 grp .. 64 grp + 63).
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
  // and their 32-term sums stay inside fp16 range. Rows >= m_rows are staged
  // as zeros with scale 1, so the main kernel runs every row unpredicated.
  int e = 0;
  if (amax > 0.0f) {
    int E;
    (void)frexpf(amax, &E);
    e = 10 - E;
    e = e > 100 ? 100 : e;
  }
  uint8_t *qbase = staged + q * kQuadBytes;
  if (c == 0) *(float *)(qbase + kXiOffset + 4 * m) = ldexpf(1.0f, -e);

  const int lane_s = m + 16 * bq;  // lane index of this row/block in XS
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

  // XA: group grp is read by lanes kg = 2(grp%2), 2(grp%2)+1, in k-steps
  // 0..3 (q0, grp < 2) or 4..7 (q1, grp >= 2).
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int kg = 2 * (grp & 1) + kk;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int s = (grp < 2 ? 0 : 4) + s4;
      unsigned hw[4], lw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // lane_weight_index(kg, s, i) - 64 grp: the same offset for every
        // group, which keeps the index into v[] a compile-time constant
        const int i0 = 2 * p, i1 = 2 * p + 1;
        const int base = ((s4 & 2) ? 32 : 0) + 16 * kk + 8 * (s4 & 1);
        const float x0 = v[base + (i0 & 4) + ((i0 & 1) << 1) + ((i0 >> 1) & 1)];
        const float x1 = v[base + (i1 & 4) + ((i1 & 1) << 1) + ((i1 >> 1) & 1)];
        _Float16 a0 = (_Float16)x0, a1 = (_Float16)x1;
        _Float16 b0 = (_Float16)(x0 - (float)a0), b1 = (_Float16)(x1 - (float)a1);
        half2v ha = {a0, a1}, hb = {b0, b1};
        hw[p] = as_u(ha);
        lw[p] = as_u(hb);
      }
      uint8_t *dst = qbase + (int64_t)bq * kXaBlockBytes + (int64_t)(s * 2) * 1024 + (m + 16 * kg) * 16;
      *(u32x4 *)dst = u32x4{hw[0], hw[1], hw[2], hw[3]};
      *(u32x4 *)(dst + 1024) = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
  }
}

// ---------------------------------------------------------------------------

__global__ void kq_fill_kernel(unsigned *p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Main kernel. A workgroup of W waves owns R = 16 T W consecutive output rows
// of one matrix (blockIdx.x = matrix * n_wg_per + row group) and the quads
// [qps blockIdx.y, +qps) of k. Wave w processes the T 16-row tiles t W + w
// (t < T); the activations of each block are staged once in LDS per
// workgroup and every A-operand read from LDS feeds all T tiles of the wave,
// so both the activation traffic and the LDS reads per weight byte fall as
// 1/T (and the staging as 1/W). Every tile runs exactly the arithmetic of a
// one-tile wave, so results do not depend on W or T.

struct WTile {
  u32x4 hdr, q0, q1;
};

template <int W, int T>
__global__ __launch_bounds__(64 * W) void kq_gemv_kernel(GemvLaunch a) {
  constexpr int kNth = 64 * W;
  constexpr int kRows = 16 * T * W;
  constexpr int kXj = (int)(kXaBlockBytes / 16) / kNth;  // 16-B activation chunks per thread per block
  static_assert(kXj * 16 * kNth == kXaBlockBytes, "activation block must split evenly");
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
  const int wg = blockIdx.x;
  const int mat = wg / a.g.n_wg_per;
  const int wgl = wg - mat * a.g.n_wg_per;
  const int64_t row0 = (int64_t)wgl * kRows;
  int64_t row[T];
  const uint8_t *rowp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    row[t] = row0 + (int64_t)(t * W + wave) * 16 + ln;
    rowp[t] = a.w[mat] + (row[t] < N ? row[t] : N - 1) * a.row_bytes;
  }

  const int q_begin = blockIdx.y * a.g.qps;
  const int q_end = min(a.g.quads, q_begin + a.g.qps);
  const int64_t b_begin = (int64_t)q_begin * 4;
  const int64_t b_last = min(KB, (int64_t)q_end * 4) - 1;  // last block of this split

  const unsigned mask_lo = in_vgpr(0x000F000Fu);
  const unsigned mask_hi = in_vgpr(0x00F000F0u);
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline. The weights rotate through four register sets (the
  // quad loop is unrolled four times, one step per block) so that the loads
  // of block b+3 are in flight while block b computes; the activations of
  // block b+2 are loaded during block b and written to LDS at the end of
  // block b+1. Every load is unconditional (indices are clamped to the
  // split's last block) so that outstanding loads are counted statically and
  // each wait covers only the data about to be used.
  auto clampb = [&](int64_t b) -> int64_t { return b < b_last ? b : b_last; };
  auto load_w = [&](WTile(&w)[T], int64_t b) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint8_t *p = rowp[t] + b * kBlockBytes;
      w[t].hdr = ld16(p);
      w[t].q0 = ld16(p + 16 + 16 * kg);
      w[t].q1 = ld16(p + 80 + 16 * kg);
    }
  };
  auto x_src = [&](int64_t b) -> const uint8_t * {
    return a.staged + (b >> 2) * kQuadBytes + (b & 3) * kXaBlockBytes;
  };
  auto load_x = [&](u32x4(&xr)[kXj], int64_t b) {
    const uint8_t *src = x_src(b);
#pragma unroll
    for (int j = 0; j < kXj; ++j) xr[j] = ld16(src + (tid + kNth * j) * 16);
  };
  WTile w0[T], w1[T], w2[T], w3[T];
  load_w(w0, b_begin);
  load_w(w1, clampb(b_begin + 1));
  load_w(w2, clampb(b_begin + 2));
  u32x4 xr0[kXj], xr1[kXj];
  load_x(xr0, b_begin);
  load_x(xr1, clampb(b_begin + 1));
#pragma unroll
  for (int j = 0; j < kXj; ++j) *(u32x4 *)(&s_x[0][(tid + kNth * j) * 16]) = xr0[j];
  __syncthreads();

  for (int q = q_begin; q < q_end; ++q) {
    const uint8_t *qb = a.staged + (int64_t)q * kQuadBytes;
    const u32x4 xs_hi = ld16(qb + kXsOffset + lane * 16);
    const u32x4 xs_lo = ld16(qb + kXsOffset + 1024 + lane * 16);
    const f32x4 xinv = *(const f32x4 *)(qb + kXiOffset + 16 * kg);
    const int64_t qb0 = (int64_t)q * 4;
    const int nblk = (int)(min((int64_t)4, b_last + 1 - qb0));
    f32x4 G[T];
    u32x4 hmin[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      G[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      hmin[t] = u32x4{0u, 0u, 0u, 0u};
    }

    // One block: prefetch the activations of block b+2 (into xl) and the
    // weights of block b+3 (into pf), contract the weights in `cur` with the
    // activations in LDS buffer bq&1, then move the activations of block b+1
    // (loaded one step earlier, in xw) into the other LDS buffer.
    auto step = [&](WTile(&cur)[T], WTile(&pf)[T], u32x4(&xl)[kXj], u32x4(&xw)[kXj], const int bq) {
      const int64_t b = qb0 + bq;
      load_x(xl, clampb(b + 2));
      load_w(pf, clampb(b + 3));
      __builtin_amdgcn_sched_barrier(0);
      if (bq < nblk) {
        // per tile: block scale d and the four sub-block scales this lane
        // applies. q0 holds sub-blocks 2(kg>>1) (low nibbles) and 2(kg>>1)+1
        // (high); q1 holds 4+2(kg>>1) and 5+2(kg>>1).
        float d[T];
        half2v m00[T], c00[T], m01[T], c01[T], m10[T], c10[T], m11[T], c11[T];
        const int sh = (kg >> 1) * 16;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const u32x4 h = cur[t].hdr;
          hmin[t] = bq == kg ? h : hmin[t];
          d[t] = h2f_lo(h.x);
          const unsigned sc03 = h.y & 0x3F3F3F3Fu;
          const unsigned sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
          const float s00 = (float)((sc03 >> sh) & 0xFFu);
          const float s01 = (float)((sc03 >> (sh + 8)) & 0xFFu);
          const float s10 = (float)((sc47 >> sh) & 0xFFu);
          const float s11 = (float)((sc47 >> (sh + 8)) & 0xFFu);
          // low nibble q: (1024 + q) s - 1024 s; high nibble: (1024 + 16q) s/16 - 64 s
          m00[t] = half2v{(_Float16)s00, (_Float16)s00};
          c00[t] = half2v{(_Float16)(-1024.0f * s00), (_Float16)(-1024.0f * s00)};
          m01[t] = half2v{(_Float16)(0.0625f * s01), (_Float16)(0.0625f * s01)};
          c01[t] = half2v{(_Float16)(-64.0f * s01), (_Float16)(-64.0f * s01)};
          m10[t] = half2v{(_Float16)s10, (_Float16)s10};
          c10[t] = half2v{(_Float16)(-1024.0f * s10), (_Float16)(-1024.0f * s10)};
          m11[t] = half2v{(_Float16)(0.0625f * s11), (_Float16)(0.0625f * s11)};
          c11[t] = half2v{(_Float16)(-64.0f * s11), (_Float16)(-64.0f * s11)};
        }
        f32x4 chi[T], clo[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          chi[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          clo[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const uint8_t *xb = s_x[bq & 1];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const half8 ahi = *(const half8 *)(xb + (s * 2 + 0) * 1024 + lane * 16);
          const half8 alo = *(const half8 *)(xb + (s * 2 + 1) * 1024 + lane * 16);
          const bool hi = (s & 2) != 0;
          const unsigned mask = hi ? mask_hi : mask_lo;
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const u32x4 qq = s < 4 ? cur[t].q0 : cur[t].q1;
            const unsigned da = (s & 1) ? qq.z : qq.x;
            const unsigned db = (s & 1) ? qq.w : qq.y;
            const half2v sc = s < 4 ? (hi ? m01[t] : m00[t]) : (hi ? m11[t] : m10[t]);
            const half2v nb = s < 4 ? (hi ? c01[t] : c00[t]) : (hi ? c11[t] : c10[t]);
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
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) G[t][r] += d[t] * (chi[t][r] + clo[t][r]);
      }
#pragma unroll
      for (int j = 0; j < kXj; ++j) *(u32x4 *)(&s_x[(bq & 1) ^ 1][(tid + kNth * j) * 16]) = xw[j];
      __syncthreads();
    };
    step(w0, w3, xr0, xr1, 0);
    step(w1, w0, xr1, xr0, 1);
    step(w2, w1, xr0, xr1, 2);
    step(w3, w2, xr1, xr0, 3);

    // end of the quad: min term (three MFMAs per tile) and the row scale
    // 2^-e. Lane kg supplies dmin * m_j of block kg of the quad in k-slots
    // 8kg..8kg+7; the A operand holds the matching scaled sub-block sums.
    const half8 a2h = __builtin_bit_cast(half8, xs_hi);
    const half8 a2l = __builtin_bit_cast(half8, xs_lo);
    const bool ok = kg < nblk;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const u32x4 h = hmin[t];
      const float dmin = h2f_hi(h.x);
      const unsigned m03 = h.z & 0x3F3F3F3Fu;
      const unsigned m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
      unsigned bh[4], bl[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const unsigned src = p < 2 ? m03 : m47;
        const int shp = (p & 1) * 16;
        const float v0 = ok ? dmin * (float)((src >> shp) & 0xFFu) : 0.0f;
        const float v1 = ok ? dmin * (float)((src >> (shp + 8)) & 0xFFu) : 0.0f;
        const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
        const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
        half2v hh = {h0, h1}, ll = {l0, l1};
        bh[p] = as_u(hh);
        bl[p] = as_u(ll);
      }
      const half8 b2h = make_h8(bh[0], bh[1], bh[2], bh[3]);
      const half8 b2l = make_h8(bl[0], bl[1], bl[2], bl[3]);
      f32x4 c2 = {0.f, 0.f, 0.f, 0.f};
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2h, b2h, c2, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2l, b2h, c2, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2h, b2l, c2, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] += xinv[r] * (G[t][r] - c2[r]);
    }
  }

  // ---------------------------------------------------------------- epilogue
  // lane holds acc[t][r] = logit of activation row 4kg+r, output row row[t]
  const int splits = a.g.splits;
  float *logits = a.logits[mat];

  if (tid < kMaxRows) s_keys[tid] = 0ull;

  if (splits == 1) {
    if (logits) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (row[t] < N) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = 4 * kg + r;
            if (m < M) logits[(int64_t)m * N + row[t]] = acc[t][r];
          }
        }
      }
    }
    if (a.verify) {
      __syncthreads();
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (row[t] < N) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = 4 * kg + r;
            if (m < M) atomicMax(&s_keys[m], argmax_key(acc[t][r], (unsigned)row[t]));
          }
        }
      }
    }
  } else {
    // write this split's partial sums, then the last arriving split sums all
    // splits in split order.
    float *part = a.partials + ((int64_t)blockIdx.y * a.g.count + mat) * kMaxRows * N;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (row[t] < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * kg + r;
          if (m < M) st_dev(&part[(int64_t)m * N + row[t]], acc[t][r]);
        }
      }
    }
    stores_done_barrier();
    if (tid == 0) {
      const unsigned old =
          __hip_atomic_fetch_add(&a.tile_cnt[wg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == (unsigned)(splits - 1);
      if (last) __hip_atomic_store(&a.tile_cnt[wg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = last;
    }
    __syncthreads();
    if (!s_flag) return;
    // Sum the splits in split order. Thread i handles row i % kRows of the
    // group for activation rows i / kRows, +kNth / kRows, ...; all loads of
    // a chunk of splits are issued before the first is used.
    const int nrows = (int)min((int64_t)kRows, N - row0);
    const int64_t split_stride = (int64_t)a.g.count * kMaxRows * N;
    const float *p0 = a.partials + (int64_t)mat * kMaxRows * N;
    constexpr int kChunk = 8;
    for (int i = tid; i < kRows * kMaxRows; i += kNth) {
      const int m = i / kRows;
      const int r = i % kRows;
      if (m >= M || r >= nrows) continue;
      const int64_t n = row0 + r;
      const float *src = p0 + (int64_t)m * N + n;
      float v = 0.0f;
      for (int sp0 = 0; sp0 < splits; sp0 += kChunk) {
        float pv[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c)
          pv[c] = sp0 + c < splits ? ld_dev(src + (int64_t)(sp0 + c) * split_stride) : 0.0f;
#pragma unroll
        for (int c = 0; c < kChunk; ++c)
          if (sp0 + c < splits) v = sp0 + c == 0 ? pv[c] : v + pv[c];
      }
      if (logits) logits[(int64_t)m * N + n] = v;
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
      for (int w = tid >> 4; w < a.g.n_wg; w += kNth / 16) {
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
  const dim3 grid((unsigned)a.g.n_wg, (unsigned)a.g.splits);
  hipStream_t st = (hipStream_t)stream;
  switch (a.g.waves * 16 + a.g.tpw) {
    case 4 * 16 + 1: hipLaunchKernelGGL((kq_gemv_kernel<4, 1>), grid, dim3(256), 0, st, a); break;
    case 4 * 16 + 2: hipLaunchKernelGGL((kq_gemv_kernel<4, 2>), grid, dim3(256), 0, st, a); break;
    case 4 * 16 + 4: hipLaunchKernelGGL((kq_gemv_kernel<4, 4>), grid, dim3(256), 0, st, a); break;
    case 8 * 16 + 1: hipLaunchKernelGGL((kq_gemv_kernel<8, 1>), grid, dim3(512), 0, st, a); break;
    case 8 * 16 + 2: hipLaunchKernelGGL((kq_gemv_kernel<8, 2>), grid, dim3(512), 0, st, a); break;
    default: return (int)hipErrorInvalidConfiguration;
  }
  return (int)hipGetLastError();
}

}  // namespace kq
