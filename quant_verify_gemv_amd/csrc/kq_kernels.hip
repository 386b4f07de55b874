// kq_kernels.hip -- HIP kernels for the Q4_K batched verify step on gfx950.
//
//  * kq_stage_kernel: fp32 activation rows -> the MFMA operand format, one
//    record per 256-column block: per row a power-of-two scale 2^e from the
//    row's largest magnitude in the block, every scaled value split into an
//    fp16 pair hi + lo (|x - hi - lo| <= 2^-22 |x| in range), laid out in the
//    lane order the weight unpack produces, plus the scaled 32-column
//    sub-block sums the min term needs.
//  * kq_gemv_kernel: persistent workgroups each walk an equal, contiguous run
//    of (row group, 256-column block) units. Each wave owns T 16-row tiles of
//    the row group; it streams their 144-byte super-blocks once for all
//    activation rows, unpacks the 4-bit quants times their 6-bit sub-block
//    scale into exact fp16 (q * sc <= 945) and contracts them with the staged
//    rows on v_mfma_f32_16x16x32_f16 (16 activation rows x 16 outputs x 32
//    columns); the min term -dmin * m_j * (sum of x over sub-block j) is one
//    v_mfma_f32_16x16x16_f16 per block with the exact 6-bit m_j as the B
//    operand. Block scale d, dmin and the row scale 2^-e are applied in fp32.
//    A row group that is split between workgroups is summed in fixed
//    workgroup order by the last contributor to arrive; in verify mode every
//    workgroup also takes the row argmax (ties -> lowest index) of the rows it
//    finished and the last workgroup applies the greedy accept rule.
//  * kq_fill_kernel: zeroes control words.
//
// The format (muser-book ch. 8 "The DFlash draft", section 8.2) and the
// accept rule (ch. 33 "Speculation: the local win and the distributed
// verdict", section 33.2, temperature-0 limit) are described in kq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kq_internal.h"

namespace kq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
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

// a * k.x + k.y on both halves of a: the compiler makes it one
// v_pk_fma_f16 whose op_sel modifiers broadcast the two halves of k, so each
// {scale, offset} pair occupies a single register. (Compiler builtins, not
// inline asm, for every value that feeds an MFMA: the compiler inserts the
// wait states between a VALU write and an MFMA read only for instructions
// it can see; an inline-asm product feeding the Q6_K operand once read a
// stale register under a two-tile schedule.)
__device__ __forceinline__ half2v fma_bcast(half2v a, half2v k) {
  return __builtin_elementwise_fma(a, half2v{k[0], k[0]}, half2v{k[1], k[1]});
}

// a * b and a * b - c on fp16 pairs, rounded exactly once each (v_pk_mul_f16
// with contraction off, v_pk_fma_f16): the Q6_K operand split needs the
// rounded product and its exact remainder.
__device__ __forceinline__ half2v pk_mul(half2v a, half2v b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ half2v pk_fma_sub(half2v a, half2v b, half2v c) {
  return __builtin_elementwise_fma(a, b, -c);
}

// (h >> from) & mask, moved to start at bit `to` (from, to compile-time).
__device__ __forceinline__ unsigned bit_move(unsigned h, int from, unsigned mask, int to) {
  return to >= from ? (h << (to - from)) & (mask << to) : (h >> (from - to)) & (mask << to);
}

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
// Raw buffer resource over [base, base + 4 GiB): loads and stores through
// it take a 32-bit lane offset and a 32-bit uniform offset, so no 64-bit
// address arithmetic per access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)0xFFFFFFFFu, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// Weight loads: every byte is read once per call. Tiled records are whole
// cache lines read once, so they carry the nontemporal (streaming) cache
// policy; the activations, which every workgroup re-reads, keep the
// default. So do weights in llama.cpp rows: a 144-byte block shares its
// first and last 128-byte lines with the neighbouring blocks of its row,
// which the next unit reads about a microsecond later, and a streamed line
// is gone by then (the 52-layer chain over rows is 20 % faster with the
// default policy, the tiled chain 3 % slower).
constexpr int kCpolNt = 2;
__device__ __forceinline__ u32x4 buf_ld16_w(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCpolNt));
}
// the three 16-byte weight loads of a Q4_K tile (header, two quant halves),
// streamed for the tiled layout, cached for llama.cpp rows
template <class WT>
__device__ __forceinline__ void load_q4_tile(WT &w, __amdgpu_buffer_rsrc_t r, const unsigned (&voff)[3], unsigned soff,
                                             bool tiled) {
  if (tiled) {
    w.hdr = buf_ld16_w(r, voff[0], soff);
    w.q0 = buf_ld16_w(r, voff[1], soff);
    w.q1 = buf_ld16_w(r, voff[2], soff);
  } else {
    w.hdr = buf_ld16(r, voff[0], soff);
    w.q0 = buf_ld16(r, voff[1], soff);
    w.q1 = buf_ld16(r, voff[2], soff);
  }
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 buf_ld8_w(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kCpolNt));
}
__device__ __forceinline__ unsigned buf_ld4_w(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kCpolNt);
}
__device__ __forceinline__ unsigned buf_ld2_w(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, kCpolNt);
}
// 16-byte versions for the partial sums: buffer instructions with the same
// cache policy (sc1) as the agent-scope atomic accesses above
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ void st_dev16(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCpolSc1);
}
__device__ __forceinline__ f32x4 ld_dev16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1));
}
// wait until this thread's global stores have completed, then barrier
__device__ __forceinline__ void stores_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
}

// Max of a 64-bit key over the lanes l ^ off for off = first, 2 first, ...
// below width (first = 1: the aligned group of `width` lanes).
__device__ __forceinline__ unsigned long long lanes_max(unsigned long long v, int width, int first = 1) {
  for (int off = first; off < width; off <<= 1) {
    const unsigned long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
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
// in the byte order {0,2,1,3,4,6,5,7} that the unpack produces. Column
// 64g + 32h + l of a block (g < 4, h < 2, l < 32) is quant byte 32g + l,
// nibble h, so it sits in k-step (g < 2 ? 0 : 4) + 2h + ((l>>3)&1), lane
// group kg = 2(g&1) + (l>>4), slot perm(l&7) with perm = {0,2,1,3,4,6,5,7}
// (its own inverse). The staging kernel writes the activations in exactly
// this order.
//
// Min term. For 16x16x16 MFMA k-slot 4kg + j (j < 4) the lane holds
// sub-block 4(kg&1) + {0,2,1,3}[j]; kg < 2 carries the hi halves of the
// scaled sub-block sums, kg >= 2 the lo halves, and the B operand carries
// the 6-bit m of the same sub-blocks (kg and kg+2 alike), so one MFMA gives
// sum_j (S_hi + S_lo)_j * m_j.
__device__ __forceinline__ constexpr int perm8(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }

// ---------------------------------------------------------------------------
// Staging. One workgroup per 256-column block and 16-row slice (grid:
// blocks x slices, records [block][slice]); thread t handles row
// 16 slice + t/16 (record row m = t/16) and the 16 columns [16c, 16c+16) of
// the block, c = t%16.
__global__ __launch_bounds__(256) void kq_stage_kernel(const float *__restrict__ x, int m_rows,
                                                       int64_t k, uint8_t *__restrict__ staged,
                                                       unsigned *__restrict__ ctrl,
                                                       int64_t n_groups) {
  const int t = threadIdx.x;
  const int m = t >> 4;
  const int c = t & 15;
  const int64_t b = blockIdx.x;
  const int slice = blockIdx.y;
  const int mg = 16 * slice + m;     // activation row
  const bool active = mg < m_rows;  // rows >= m_rows are staged as zeros

  if (ctrl && b == 0 && slice == 0) {
    if (t == 0) ctrl[0] = 0u;
    for (int64_t i = t; i < n_groups; i += 256) ctrl[kCntOff / 4 + i * kCntStride] = 0u;
  }

  float v[16];
  float amax = 0.0f;
  if (active) {
    const f32x4 *src = (const f32x4 *)(x + (int64_t)mg * k + b * kQK + 16 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 f = src[i];
      v[4 * i + 0] = f[0]; v[4 * i + 1] = f[1]; v[4 * i + 2] = f[2]; v[4 * i + 3] = f[3];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
  }
  // max over the 16 threads of row m (16 consecutive lanes of one wave)
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));

  // 2^e puts the row's largest magnitude in the block in [2^9, 2^10):
  // scaled values and their 32-term sums stay inside fp16 range.
  int e = 0;
  if (amax > 0.0f) {
    int E;
    (void)frexpf(amax, &E);
    e = 10 - E;
    e = e > 100 ? 100 : e;
  }
  uint8_t *rec = staged + (b * gridDim.y + slice) * kStageBytes;
  if (c == 0) *(float *)(rec + kXiOffset + 4 * m) = ldexpf(1.0f, -e);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = ldexpf(v[i], e);

  // sub-block sb = c/2 holds columns [32 sb, 32 sb + 32): this thread's 16
  // plus its neighbour's (lane t^1)
  float ssum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ssum += v[i];
  ssum += __shfl_xor(ssum, 1, 16);
  if ((c & 1) == 0) {
    const int sb = c >> 1;
    const int slot = ((sb & 1) << 1) | ((sb >> 1) & 1);  // position of sb&3 in {0,2,1,3}
    const _Float16 hi = (_Float16)ssum;
    const _Float16 lo = (_Float16)(ssum - (float)hi);
    _Float16 *xsb = (_Float16 *)(rec + kXsbOffset);
    xsb[(m + 16 * (sb >> 2)) * 4 + slot] = hi;
    xsb[(m + 16 * (2 + (sb >> 2))) * 4 + slot] = lo;
  }

  // XA: columns 16c + j sit in k-step s0 + (j >> 3), lane m + 16 kg, slot
  // perm8(j & 7) (see the lane-order note above).
  const int g = c >> 2, h = (c >> 1) & 1;
  const int kg = 2 * (g & 1) + (c & 1);
  const int s0 = (g < 2 ? 0 : 4) + 2 * h;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    unsigned hw[4], lw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = v[8 * hh + perm8(2 * p)];
      const float x1 = v[8 * hh + perm8(2 * p + 1)];
      const _Float16 a0 = (_Float16)x0, a1 = (_Float16)x1;
      const _Float16 b0 = (_Float16)(x0 - (float)a0), b1 = (_Float16)(x1 - (float)a1);
      const half2v ha = {a0, a1}, hb = {b0, b1};
      hw[p] = as_u(ha);
      lw[p] = as_u(hb);
    }
    uint8_t *dst = rec + (int64_t)((s0 + hh) * 2) * 1024 + (m + 16 * kg) * 16;
    *(u32x4 *)dst = u32x4{hw[0], hw[1], hw[2], hw[3]};
    *(u32x4 *)(dst + 1024) = u32x4{lw[0], lw[1], lw[2], lw[3]};
  }
}

// ---------------------------------------------------------------------------

__global__ void kq_fill_kernel(unsigned *p, int64_t n, unsigned value) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = value;
}

// ---------------------------------------------------------------------------
// Main kernel. Persistent workgroup p of W waves walks the units
// [u0, u0 + nu) in row-group-major order (unit u = row group u / kb, block
// u % kb). Wave w owns the T 16-row tiles t W + w of the current row group;
// the activations of each block are staged once in LDS per workgroup and
// every A-operand read from LDS feeds all T tiles of the wave.

// One 16-row tile's share of a block in a lane's registers: Q4_K and Q5_K
// header, two quant chunks; Q5_K fifth bits in hx.x, hx.y; Q6_K: scale
// dword in hdr.x, d in hdr.y, low nibbles in q0, q1, high parts in hx.
struct WTile {
  u32x4 hdr, q0, q1, hx;
};
__device__ __forceinline__ unsigned sel4(const u32x4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

constexpr int lcm_int(int a, int b) {
  int x = a, y = b;
  while (y) {
    const int r = x % y;
    x = y;
    y = r;
  }
  return a / x * b;
}

// Grid barrier between the phases of a chain launch (kq_chain_kernel). Every
// workgroup adds one arrival to a
// device-wide count (agent-scope atomic); the phase is complete when the
// count reaches (phase + 1) times the workgroups. The workgroup whose
// arrival completes the count releases the others: its threads write every
// workgroup's own release flag, one 256-byte line per workgroup, and each
// waiting workgroup polls only its own flag. (Polling the count itself from
// every workgroup, one hot line, was measured to slow the last workgroups'
// own coherent stores and atomics, the split-group reductions, severalfold.)
// A flag holds (launch epoch << 32) | (barrier + 1), so a flag left by the
// previous launch never matches; the epoch is a device word the final
// arrival of each launch increments, read by every workgroup before its
// first arrival. Every wait gives up after kSpinTicks of the 100 MHz
// real-time counter (or when another workgroup has raised *err) and raises
// *err, so every wait ends.
constexpr unsigned long long kSpinTicks = 100000000ull;  // 1 s
constexpr int kFlagStride = 32;                        // u64 words between release flags (256 bytes)

__device__ __forceinline__ int spin_flag(const unsigned long long *flag, unsigned long long want, unsigned *err) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    if (ld_dev(flag) == want) return 1;
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return 0;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return 0;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Field f of the launch's phase.
#define KQ_PH(I_, f) (a.ph.f)

// ROWS: Q4_K weights in llama.cpp rows (else the tiled layout); a template
// parameter so that the weight loads' cache policy is fixed at compile time
template <int W, int T, int BI, int D, int FMT, int MS, bool ROWS>
__global__ __launch_bounds__(64 * W, W == 4 ? (T == 1 ? 3 : 2) : 1) void kq_gemv_kernel(GemvLaunch a) {
  static_assert(W % 4 == 0, "waves spread evenly over the 4 SIMDs");
  static_assert(!ROWS || FMT == kFmtQ4, "only Q4_K has a row-layout path");
  // MS 16-row activation slices: every unpacked weight operand feeds the
  // MFMAs of all MS slices, so the weights are read once for 16 MS rows
  static_assert(MS >= 1 && MS <= 4, "one to four slices per launch");
  constexpr int kRS = 16 * MS;  // activation rows per call at most
  constexpr unsigned kTB = 16u * (unsigned)fmt_block_bytes(FMT);  // tiled record bytes
  // D weight register sets: the weights of unit i + D - 1 are loaded while
  // unit i computes. The activations of unit i + BI are stored to LDS in
  // step i from registers loaded kXL steps earlier: loads complete in issue
  // order, so waiting for them waits only for weights issued before step
  // i - kXL, which step i needs anyway when kXL >= D - 2. Four-wave
  // workgroups stage twice the activation chunks per thread and keep one
  // set in flight. The unit loop is unrolled kU = lcm(D, BI, kXL + 1) times
  // so that every register set index and every interval position is static.
  // Three or four slices: the activations of unit i + 1 are copied into LDS
  // by direct-to-LDS buffer loads issued in step i (kDma, no register
  // staging, so the two-tile waves stay within their 256 registers); the
  // workgroup barrier that ends step i waits for them. The ring's two
  // halves are indexed statically, so the compiler sees that a copy into
  // one half never aliases the reads of the other.
  constexpr bool kDma = MS >= 3;
  constexpr int kXL = (W >= 8 && T == 1 && MS == 1) ? 3 : kDma ? 0 : 1;
  constexpr int kU = lcm_int(lcm_int(D, BI), kXL + 1);
  constexpr int kNth = 64 * W;
  constexpr int kRows = 16 * T * W;
  // The staged record is kXc 16-byte chunks, copied linearly; thread tid
  // moves chunks tid + j kNth (the last round only partly).
  constexpr int kXc = (int)(kStageBytes * MS / 16);  // 1,060 per slice
  constexpr int kXj = (kXc + kNth - 1) / kNth;   // chunks per thread
  // Activation ring: unit i sits in buffer i % kNB. Workgroups synchronise
  // once every BI units: between two barriers the waves read BI buffers and
  // fill the other BI.
  constexpr int kNB = 2 * BI;
  static_assert(BI == 1 || BI == 2 || BI == 4, "barrier interval");
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kNB][kStageBytes * MS];
  __shared__ unsigned long long s_keys[kRS];
  __shared__ int s_am[kMaxTreeRows];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kg = lane >> 4;
  const int ln = lane & 15;
  const int M = a.m;
  // unit indices fit in 32 bits: every matrix is smaller than 4 GiB, so a
  // phase has fewer than 2^31 units
  const int P = gridDim.x;
  const int p = blockIdx.x;

  // this workgroup's run of the U units of a phase
  auto run_start = [&](int U) -> int {
    const int b = U / P, r = U % P;
    return p * b + (p < r ? p : r);
  };
  auto run_len = [&](int U) -> int { return U / P + (p < U % P ? 1 : 0); };
  auto tile_row = [&](int t) -> int { return (t * W + wave) * 16 + ln; };  // row within the group

  if (tid < kRS) s_keys[tid] = 0ull;

  const unsigned mask_lo = in_vgpr(0x000F000Fu);
  // byte-permute selector that puts this lane's two scale bytes 2(kg>>1),
  // 2(kg>>1)+1 of a packed word into the low bytes of an fp16 pair
  const unsigned sel_sc = (kg >> 1) ? 0x00070006u : 0x00050004u;
  const unsigned mask_hi = in_vgpr(0x00F000F0u);

  // Weight stream: the weights run D - 1 units ahead of the compute,
  // clamped to the launch's last unit, so every load is unconditional and
  // outstanding loads are counted statically.
  // Addressing, one code path for both layouts, through buffer loads from
  // the current matrix (every matrix is smaller than 4 GiB): the lane's
  // bytes of block b of tile t sit at voff[t][0..2] + soff[t] + b *
  // block_stride. Row-major (llama.cpp): voff = the lane's row (clamped to
  // the last row) times the row bytes + {0, 16 + 16kg, 80 + 16kg}, soff = 0,
  // stride 144. Tiled: voff = {16 ln, 256 + 16 lane, 1,280 + 16 lane}, soff
  // = the 16-row tile's record, stride = tiles * 2,304.
  constexpr bool tiled = !ROWS;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int uw = 0, uw_last = 0, gw = 0, bw = 0;
  auto w_n = [&]() -> int { return a.ph.n; };
  auto w_rb = [&]() -> int { return a.ph.row_bytes; };
  auto w_nt = [&]() -> int { return a.ph.n_tiles; };
  auto w_kb = [&]() -> int { return a.ph.kb; };
  auto w_nwg = [&]() -> int { return a.ph.n_wg_per; };
  auto block_stride = [&]() -> unsigned {
    return tiled ? (unsigned)w_nt() * kTB : (unsigned)kBlockBytes;
  };
  unsigned boff = 0;
  __amdgpu_buffer_rsrc_t w_rsrc;
  unsigned voff[T][3], soff[T];
  auto set_rowp = [&]() {
    const int mat = gw / w_nwg();
    const int r0 = (gw - mat * w_nwg()) * kRows;
    w_rsrc = dev_rsrc(KQ_PH(wp, w[mat]));
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (tiled) {
        int ti = (r0 + (t * W + wave_u) * 16) / 16;
        ti = ti < w_nt() ? ti : w_nt() - 1;
        soff[t] = (unsigned)ti * kTB;
        voff[t][0] = 16u * ln;
        voff[t][1] = (unsigned)kTileQ0 + 16u * lane;
        voff[t][2] = (unsigned)kTileQ1 + 16u * lane;
      } else {
        const int row = r0 + tile_row(t);
        const unsigned rb = (unsigned)(row < w_n() ? row : w_n() - 1) * (unsigned)w_rb();
        soff[t] = 0u;
        voff[t][0] = rb;
        voff[t][1] = rb + 16u + 16u * kg;
        voff[t][2] = rb + 80u + 16u * kg;
      }
    }
  };
  auto begin_w = [&](int ph) {
    const int U = KQ_PH(ph, units);
    uw = run_start(U);
    uw_last = uw + run_len(U) - 1;
    gw = uw / w_kb();
    bw = uw % w_kb();
    boff = (unsigned)bw * block_stride();
    set_rowp();
  };
  auto load_w = [&](WTile(&w)[T]) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (FMT == kFmtQ4) {
        load_q4_tile(w[t], w_rsrc, voff[t], soff[t] + boff, tiled);
      } else {
        if constexpr (FMT == kFmtQ6) {
          w[t].hdr.x = buf_ld4_w(w_rsrc, 4u * lane, soff[t] + boff);
          w[t].hdr.y = buf_ld2_w(w_rsrc, (unsigned)kTileQ6D + 2u * ln, soff[t] + boff);
        } else {
          w[t].hdr = buf_ld16_w(w_rsrc, voff[t][0], soff[t] + boff);
        }
        w[t].q0 = buf_ld16_w(w_rsrc, voff[t][1], soff[t] + boff);
        w[t].q1 = buf_ld16_w(w_rsrc, voff[t][2], soff[t] + boff);
      }
      if constexpr (FMT == kFmtQ5) {
        const u32x2 h = buf_ld8_w(w_rsrc, (unsigned)kTileQH + 8u * lane, soff[t] + boff);
        w[t].hx.x = h.x;
        w[t].hx.y = h.y;
      }
      if constexpr (FMT == kFmtQ6) w[t].hx = buf_ld16_w(w_rsrc, (unsigned)kTileQH + 16u * lane, soff[t] + boff);
    }
    if (uw < uw_last) {
      ++uw;
      boff += block_stride();
      if (++bw == w_kb()) {
        bw = 0;
        boff = 0u;
        ++gw;
        set_rowp();
      }
    }
  };

  // last round: threads past the record re-load its last chunk and skip the store
  const int xlast = tid + kNth * (kXj - 1) < kXc ? tid + kNth * (kXj - 1) : kXc - 1;
  struct XRegs {
    u32x4 a[kXj];
  };
  XRegs xr[kXL + 1];
  WTile wr[D][T];
  f32x4 acc[T][MS], acc_first[T][MS];
  // finished rows of whole row groups: the argmax keys are reduced over the
  // wave's tiles and its 16 rows per lane group into a running maximum per
  // activation row 4kg + r (wave_key[r], held by every lane of the group)
  // that goes to LDS after the loop.
  unsigned long long wave_key[MS][4] = {};
  const __amdgpu_buffer_rsrc_t part_rsrc = dev_rsrc(a.partials);
  auto put = [&](float *q, float v) { *q = v; };

  begin_w(0);

  {
    [[maybe_unused]] const int ph = 0;  // single phase: KQ_PH reads the launch's own fields
    const int N = KQ_PH(ph, n);
    const int KB = KQ_PH(ph, kb);
    const int n_wg_per = KQ_PH(ph, n_wg_per);
    const int U = KQ_PH(ph, units);
    const int base = U / P, rem = U % P;
    const int u0 = p * base + (p < rem ? p : rem);
    const int nu = base + (p < rem ? 1 : 0);
    const int u_last = u0 + nu - 1;
    auto owner = [&](int u) -> int {
      const int big = rem * (base + 1);
      return u < big ? u / (base + 1) : rem + (u - big) / base;
    };
    auto group_row0 = [&](int g, int &mat) -> int {
      mat = g / n_wg_per;
      return (g - mat * n_wg_per) * kRows;
    };
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int sl = 0; sl < MS; ++sl) {
        acc[t][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_first[t][sl] = acc[t][sl];
      }

    // Activation stream, two units behind the weights and never past the
    // launch's last unit.
    int ux = u0;
    int bx = u0 % KB;
    const __amdgpu_buffer_rsrc_t x_rsrc = dev_rsrc(KQ_PH(ph, staged));
    const unsigned x_rec = a.x_rec;
    auto load_x = [&](XRegs &x) {
      const unsigned src = (unsigned)bx * x_rec;
#pragma unroll
      for (int j = 0; j < kXj; ++j)
        x.a[j] = buf_ld16(x_rsrc, (unsigned)(j < kXj - 1 ? tid + kNth * j : xlast) * 16u, src);
      if (ux < u_last) {
        ++ux;
        if (++bx == KB) bx = 0;
      }
    };
    auto store_x = [&](int buf, const XRegs &x) {
#pragma unroll
      for (int j = 0; j < kXj; ++j)
        if (j < kXj - 1 || tid + kNth * j < kXc) *(u32x4 *)(&s_x[buf][(tid + kNth * j) * 16]) = x.a[j];
    };
    // buffer_load_dwordx4 ... lds: every lane's 16 bytes go straight to LDS at
    // the wave's base + 16 x lane, so instruction j of wave w copies chunks
    // kNth j + 64 w .. + 63 of the record (one contiguous KiB); lanes past
    // the record's end issue nothing. `buf` must be a compile-time constant.
    auto dma_x = [&](const int buf) {
      const unsigned src = (unsigned)bx * x_rec;
#pragma unroll
      for (int j = 0; j < kXj; ++j) {
        const int cb = kNth * j + 64 * wave_u;
        if (cb < kXc && cb + lane < kXc)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              x_rsrc, (__attribute__((address_space(3))) void *)(&s_x[buf][cb * 16]), 16,
              (unsigned)(cb + lane) * 16u, src, 0, 0);
      }
      if (ux < u_last) {
        ++ux;
        if (++bx == KB) bx = 0;
      }
    };

    auto write_rows = [&](int g, const f32x4(&v)[T][MS]) {
      int mat;
      const int r0 = group_row0(g, mat);
      float *logits = KQ_PH(ph, logits[mat]);
      if (logits) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int row = r0 + tile_row(t);
          if (row < N) {
#pragma unroll
            for (int sl = 0; sl < MS; ++sl)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int m = 16 * sl + 4 * kg + r;
                if (m < M) put(&logits[(int64_t)m * N + row], v[t][sl][r]);
              }
          }
        }
      }
      if (a.verify) {
#pragma unroll
        for (int sl = 0; sl < MS; ++sl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            unsigned long long best = 0ull;
#pragma unroll
            for (int t = 0; t < T; ++t) {
              const int row = r0 + tile_row(t);
              const unsigned long long key = row < N ? argmax_key(v[t][sl][r], (unsigned)row) : 0ull;
              best = key > best ? key : best;
            }
            best = lanes_max(best, 16);
            if constexpr (MS == 1) {
              wave_key[sl][r] = best > wave_key[sl][r] ? best : wave_key[sl][r];
            } else {
              // more rows: straight into LDS (no running maxima in registers)
              const int m = 16 * sl + 4 * kg + r;
              if (ln == 0 && m < M && best) atomicMax(&s_keys[m], best);
            }
          }
      }
    };

    // Prologue, in issue order (loads complete in issue order): the weights
    // of unit 0 (from HBM, the longest wait, needed first), the activations
    // of units 0..BI-1 (to buffers 0..BI-1 before the first barrier), the
    // weights of units 1..D-2, then the activations of units BI..BI+kXL-1,
    // which stay in registers (set u % (kXL + 1)).
    if constexpr (kDma) {
      static_assert(BI == 1 && kXL == 0 && D == 2, "direct-to-LDS ring: one unit per barrier, two register sets");
      load_w(wr[0]);
      dma_x(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): unit 0's activations are in LDS
    } else {
      XRegs xp[BI];
      load_w(wr[0]);
#pragma unroll
      for (int j = 0; j < BI; ++j) load_x(xp[j]);
#pragma unroll
      for (int d = 1; d < D - 1; ++d) load_w(wr[d]);
#pragma unroll
      for (int q = 0; q < kXL; ++q) load_x(xr[(BI + q) % (kXL + 1)]);
#pragma unroll
      for (int j = 0; j < BI; ++j) store_x(j, xp[j]);
    }
    __syncthreads();

    const int g_first = u0 / KB;
    int gc = g_first, bc = u0 % KB, seg0 = bc;
    int have_first = 0;

    // A partial is [row of the group][kRS activation rows] fp32: the lane's
    // four sums of a slice (activation rows 16 sl + 4kg .. +3 of its output
    // row) are one 16-byte store.
    auto write_partial = [&](int slot, const f32x4(&v)[T][MS]) {
      const unsigned base_off = (unsigned)((p * 2 + slot) * kRS * kRows) * 4u;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int sl = 0; sl < MS; ++sl)
          st_dev16(part_rsrc, base_off + (unsigned)(tile_row(t) * kRS + 16 * sl + 4 * kg) * 4u, v[t][sl]);
    };

    // One unit: prefetch the activations of unit i+BI+kXL (into xl) and the
    // weights of unit i+D-1 (into pf), contract the weights in `cur` with the
    // activations in LDS buffer i % kNB, then move the activations of unit
    // i+BI (in xs) into their buffer; barrier after every BI-th unit (pos is
    // the static position within the unrolled iteration).
    auto step = [&](WTile(&cur)[T], WTile(&pf)[T], XRegs &xl, const XRegs &xs, const int i,
                    const int pos) {
      // Waves w, w + 4, ... share a SIMD, and the oldest would otherwise win
      // issue every cycle and reach the barrier first; rotating the priority
      // each unit keeps them in step.
      if ((wave >> 2) == pos % (W / 4))
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
      static_assert(!kDma || kU % kNB == 0, "ring half of a step fixed by its place in the unrolled loop");
      if constexpr (kDma) {
        load_w(pf);
        dma_x((pos + BI) % kNB);
      } else {
        load_x(xl);
        load_w(pf);
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t *xb = s_x[kDma ? pos % kNB : i % kNB];
      if (i < nu) {
        if constexpr (FMT == kFmtQ6) {
          // Q6_K: w = d sc (q - 32), sc a signed 8-bit scale per 16 columns.
          // Each lane's 8 columns of a k-step share one scale (its 4 scales are
          // bytes 2 (s >> 2) + ((s >> 1) & 1) of hdr.x). The unpack gives the
          // fp16 1024 + q (low nibble steps) or 1024 + 16 q (high), minus 1056
          // or 1536 is q - 32 or 16 (q - 32) exactly; times sc or sc / 16 it
          // can need 13 significant bits, so the B operand is the rounded
          // product b_hi plus the exact remainder b_lo (0 or +-1); x_hi b_hi +
          // x_lo b_hi + x_hi b_lo leaves out x_lo b_lo, below 2^-22 of |w x|.
          float d6[T];
          half2v k6[T][4];
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const unsigned sw = cur[t].hdr.x;
            d6[t] = h2f_lo(cur[t].hdr.y);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float sv = (float)(int)(signed char)(sw >> (8 * j)) * ((j & 1) ? 0.0625f : 1.0f);
              const _Float16 hv = (_Float16)sv;
              k6[t][j] = half2v{hv, hv};
            }
          }
          f32x4 cq[T][MS];
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int sl = 0; sl < MS; ++sl) cq[t][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
          const half2v off_lo = {(_Float16)-1056.0f, (_Float16)-1056.0f};
          const half2v off_hi = {(_Float16)-1536.0f, (_Float16)-1536.0f};
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            half8 ahi[MS], alo[MS];
#pragma unroll
            for (int sl = 0; sl < MS; ++sl) {
              ahi[sl] = *(const half8 *)(xb + sl * kStageBytes + (s * 2 + 0) * 1024 + lane * 16);
              alo[sl] = *(const half8 *)(xb + sl * kStageBytes + (s * 2 + 1) * 1024 + lane * 16);
            }
            const bool hi = (s & 2) != 0;
            const unsigned mask = hi ? mask_hi : mask_lo;
            const half2v off = hi ? off_hi : off_lo;
            const int to = hi ? 8 : 4, c = 8 * (s & 1);
            const int j = 2 * (s >> 2) + ((s >> 1) & 1);
#pragma unroll
            for (int t = 0; t < T; ++t) {
              const u32x4 qq = s < 4 ? cur[t].q0 : cur[t].q1;
              const unsigned da = (s & 1) ? qq.z : qq.x;
              const unsigned db = (s & 1) ? qq.w : qq.y;
              // the two high bits of pairs (0,2), (1,3), (4,6), (5,7) sit at
              // bits c, c + 2, c + 4, c + 6 (+16) of high-part word s >> 1
              const unsigned hw = sel4(cur[t].hx, s >> 1);
              const half2v q0h = as_h2((da & mask) | bit_move(hw, c + 0, 0x00030003u, to) | 0x64006400u) + off;
              const half2v q1h = as_h2(((da >> 8) & mask) | bit_move(hw, c + 2, 0x00030003u, to) | 0x64006400u) + off;
              const half2v q2h = as_h2((db & mask) | bit_move(hw, c + 4, 0x00030003u, to) | 0x64006400u) + off;
              const half2v q3h = as_h2(((db >> 8) & mask) | bit_move(hw, c + 6, 0x00030003u, to) | 0x64006400u) + off;
              const half2v kk = k6[t][j];
              const half2v h0 = pk_mul(q0h, kk), h1 = pk_mul(q1h, kk), h2 = pk_mul(q2h, kk), h3 = pk_mul(q3h, kk);
              const half2v l0 = pk_fma_sub(q0h, kk, h0), l1 = pk_fma_sub(q1h, kk, h1);
              const half2v l2 = pk_fma_sub(q2h, kk, h2), l3 = pk_fma_sub(q3h, kk, h3);
              const half8 bhi = make_h8(as_u(h0), as_u(h1), as_u(h2), as_u(h3));
              const half8 blo = make_h8(as_u(l0), as_u(l1), as_u(l2), as_u(l3));
#pragma unroll
              for (int sl = 0; sl < MS; ++sl) {
                cq[t][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[sl], bhi, cq[t][sl], 0, 0, 0);
                cq[t][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[sl], bhi, cq[t][sl], 0, 0, 0);
                cq[t][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[sl], blo, cq[t][sl], 0, 0, 0);
              }
            }
          }
#pragma unroll
          for (int sl = 0; sl < MS; ++sl) {
            const f32x4 xinv = *(const f32x4 *)(xb + sl * kStageBytes + kXiOffset + 16 * kg);
#pragma unroll
            for (int t = 0; t < T; ++t) {
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[t][sl][r] += xinv[r] * (d6[t] * cq[t][sl][r]);
            }
          }
        } else {
          float d[T], dmin[T];
          // per sub-block {scale, offset} pairs; the fma broadcasts each half
          half2v k00[T], k01[T], k10[T], k11[T];
          half4 bm[T];
          const half2v neg1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
          const half2v lo_pair = {(_Float16)1.0f, (_Float16)-1024.0f};
          const half2v hi_pair = {(_Float16)0.0625f, (_Float16)-64.0f};
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const u32x4 h = cur[t].hdr;
            d[t] = h2f_lo(h.x);
            dmin[t] = h2f_hi(h.x);
            // q0 holds sub-blocks 2(kg>>1) (low nibbles) and 2(kg>>1)+1 (high);
            // q1 holds 4+2(kg>>1) and 5+2(kg>>1). Their 6-bit scales are bytes
            // 2(kg>>1), 2(kg>>1)+1 of sc03 and sc47; one byte permute sets each
            // below an fp16 exponent byte 0x64 (1024 + s), so {s, s'} is exact.
            const unsigned sc03 = h.y & 0x3F3F3F3Fu;
            const unsigned sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
            const half2v s0 = as_h2(__builtin_amdgcn_perm(sc03, 0x64646464u, sel_sc)) + neg1024;
            const half2v s1 = as_h2(__builtin_amdgcn_perm(sc47, 0x64646464u, sel_sc)) + neg1024;
            // low nibble q: (1024 + q) s - 1024 s; high nibble: (1024 + 16q) s/16 - 64 s
            k00[t] = half2v{s0[0], s0[0]} * lo_pair;
            k01[t] = half2v{s0[1], s0[1]} * hi_pair;
            k10[t] = half2v{s1[0], s1[0]} * lo_pair;
            k11[t] = half2v{s1[1], s1[1]} * hi_pair;
            // min-term B operand: the 6-bit m of sub-blocks 4(kg&1) + {0,2,1,3}
            const unsigned m03 = h.z & 0x3F3F3F3Fu;
            const unsigned m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
            const unsigned msrc = (kg & 1) ? m47 : m03;
            const half2v p0 = as_h2(__builtin_amdgcn_perm(msrc, 0x64646464u, 0x00060004u)) + neg1024;
            const half2v p1 = as_h2(__builtin_amdgcn_perm(msrc, 0x64646464u, 0x00070005u)) + neg1024;
            bm[t] = half4{p0[0], p0[1], p1[0], p1[1]};
          }
          // x hi and x lo products accumulate in one fp32 sum per tile and slice
          f32x4 cq[T][MS];
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int sl = 0; sl < MS; ++sl) cq[t][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            half8 ahi[MS], alo[MS];
#pragma unroll
            for (int sl = 0; sl < MS; ++sl) {
              ahi[sl] = *(const half8 *)(xb + sl * kStageBytes + (s * 2 + 0) * 1024 + lane * 16);
              alo[sl] = *(const half8 *)(xb + sl * kStageBytes + (s * 2 + 1) * 1024 + lane * 16);
            }
            const bool hi = (s & 2) != 0;
            const unsigned mask = hi ? mask_hi : mask_lo;
#pragma unroll
            for (int t = 0; t < T; ++t) {
              const u32x4 qq = s < 4 ? cur[t].q0 : cur[t].q1;
              const unsigned da = (s & 1) ? qq.z : qq.x;
              const unsigned db = (s & 1) ? qq.w : qq.y;
              const half2v kk = s < 4 ? (hi ? k01[t] : k00[t]) : (hi ? k11[t] : k10[t]);
              // Q5_K: the fifth bit of each weight, at bit 4 (low nibble) or 8
              // (high nibble, 16 q) of its fp16 half; pairs (bytes 0,2), (1,3),
              // (4,6), (5,7) of the 8 sit at bits c .. c + 3 (+16) of the lane's
              // fifth-bit word for steps s & ~3
              unsigned e0 = 0u, e1 = 0u, e2 = 0u, e3 = 0u;
              if constexpr (FMT == kFmtQ5) {
                const unsigned hw = s < 4 ? cur[t].hx.x : cur[t].hx.y;
                const int c = 4 * (s & 3), to = hi ? 8 : 4;
                e0 = bit_move(hw, c + 0, 0x00010001u, to);
                e1 = bit_move(hw, c + 1, 0x00010001u, to);
                e2 = bit_move(hw, c + 2, 0x00010001u, to);
                e3 = bit_move(hw, c + 3, 0x00010001u, to);
              }
              const unsigned u0_ = (da & mask) | e0 | 0x64006400u;
              const unsigned u1_ = ((da >> 8) & mask) | e1 | 0x64006400u;
              const unsigned u2_ = (db & mask) | e2 | 0x64006400u;
              const unsigned u3_ = ((db >> 8) & mask) | e3 | 0x64006400u;
              const half2v v0 = fma_bcast(as_h2(u0_), kk);
              const half2v v1 = fma_bcast(as_h2(u1_), kk);
              const half2v v2 = fma_bcast(as_h2(u2_), kk);
              const half2v v3 = fma_bcast(as_h2(u3_), kk);
              const half8 bw8 = make_h8(as_u(v0), as_u(v1), as_u(v2), as_u(v3));
#pragma unroll
              for (int sl = 0; sl < MS; ++sl) {
                cq[t][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[sl], bw8, cq[t][sl], 0, 0, 0);
                cq[t][sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[sl], bw8, cq[t][sl], 0, 0, 0);
              }
            }
          }
          // min term and the block's contribution in the row's scaled units
#pragma unroll
          for (int sl = 0; sl < MS; ++sl) {
            const half4 as4 = *(const half4 *)(xb + sl * kStageBytes + kXsbOffset + lane * 8);
            const f32x4 xinv = *(const f32x4 *)(xb + sl * kStageBytes + kXiOffset + 16 * kg);
#pragma unroll
            for (int t = 0; t < T; ++t) {
              const f32x4 c2 =
                  __builtin_amdgcn_mfma_f32_16x16x16f16(as4, bm[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[t][sl][r] += xinv[r] * (d[t] * cq[t][sl][r] - dmin[t] * c2[r]);
            }
          }
        }
      }
      // end of a row group's segment
      const int u = u0 + i;
      if (i < nu && (bc == KB - 1 || u == u_last)) {
        if (seg0 == 0 && bc == KB - 1) {
          write_rows(gc, acc);
        } else if (gc == g_first) {
          if constexpr (MS == 1) {
#pragma unroll
            for (int t = 0; t < T; ++t) acc_first[t][0] = acc[t][0];
          } else {
            write_partial(0, acc);  // more rows: stored now, not kept in registers
          }
          have_first = 1;
        }
        if (u != u_last) {
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int sl = 0; sl < MS; ++sl) acc[t][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
          seg0 = 0;
        }
      }
      if (i < nu && ++bc == KB) {
        bc = 0;
        ++gc;
      }
      if constexpr (kDma) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): unit i + 1's activations are in LDS
      } else {
        store_x((int)((i + BI) % kNB), xs);
      }
      if (pos % BI == BI - 1) __syncthreads();
    };

    // kU units per iteration so the register sets rotate statically; steps
    // past the last unit only keep the loads and barriers in step.
    for (int i = 0; i < nu; i += kU) {
#pragma unroll
      for (int j = 0; j < kU; ++j)
        step(wr[j % D], wr[(j + D - 1) % D], xr[(j + BI + kXL) % (kXL + 1)], xr[(j + BI) % (kXL + 1)], i + j,
             j);
    }
    __builtin_amdgcn_s_setprio(0);

    // -------------------------------------------------------------- epilogue
    // Row groups this workgroup finished only in part: its first (acc_first)
    // and its last (acc, when the last segment neither starts at block 0 nor
    // ends at the last block of a group other than the first). Each partial
    // goes to slot 0 (first group) or 1 (last group) of this workgroup; the
    // last contributor of a group to arrive sums all contributors' partials in
    // workgroup order.
    if (a.verify) {
#pragma unroll
      for (int sl = 0; sl < MS; ++sl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * sl + 4 * kg + r;
          if (ln == 0 && m < M && wave_key[sl][r]) atomicMax(&s_keys[m], wave_key[sl][r]);
        }
    }
    const int g_last = u_last / KB;
    const int last_partial = (g_last != g_first) && (u_last % KB != KB - 1);
    // Sum the partials of one or two row groups over their contributors in
    // workgroup order, the loads of both groups in flight together. Thread
    // tid handles the 16-byte chunks c = tid + j kNth of each group (row
    // c / (kRS/4) of the group, activation rows 4 (c % (kRS/4)) .. +3) and
    // issues the loads of eight contributors per group before it adds any
    // of them.
    constexpr int kE = kRows * kRS / (4 * kNth);  // chunks per thread
    constexpr int kC = 8 / MS;                     // contributors in flight (registers: 2 kE kC chunks)
    constexpr int kCR = kRS / 4;                   // chunks per output row
    static_assert(kE * 4 * kNth == kRows * kRS, "chunks must split evenly");
    struct Contributors {
      int pf, pl;  // first and last contributing workgroup
      int pf_slot;     // the first one's slot (the others use slot 0)
    };
    auto contributors = [&](int g) {
      const int ufirst = g * KB;
      Contributors c;
      c.pf = owner(ufirst);
      c.pl = owner(ufirst + KB - 1);
      // every contributor after the first starts inside g (slot 0); the first
      // used slot 1 unless its run also starts at the group's first block
      const int pf_u0 = c.pf * base + (c.pf < rem ? c.pf : rem);
      c.pf_slot = pf_u0 < ufirst ? 1 : 0;
      return c;
    };
    auto load_partials = [&](const Contributors &cb, int c0, f32x4(&pv)[kE][kC]) {
      // unconditional loads: contributors past the last one re-read it and
      // are dropped when summed
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const int q = cb.pf + c0 + c <= cb.pl ? cb.pf + c0 + c : cb.pl;
        const int slot = q == cb.pf ? cb.pf_slot : 0;
        const unsigned src = (unsigned)((q * 2 + slot) * kRS * kRows) * 4u;
#pragma unroll
        for (int j = 0; j < kE; ++j) pv[j][c] = ld_dev16(part_rsrc, src + (unsigned)(tid + j * kNth) * 16u);
      }
    };
    auto sum_partials = [&](const Contributors &cb, int c0, const f32x4(&pv)[kE][kC], f32x4(&v)[kE]) {
#pragma unroll
      for (int c = 0; c < kC; ++c)
#pragma unroll
        for (int j = 0; j < kE; ++j)
          if (cb.pf + c0 + c <= cb.pl) v[j] = c0 + c == 0 ? pv[j][c] : v[j] + pv[j][c];
    };
    // logits and argmax keys of a reduced group (elements past M or the
    // matrix end are dropped)
    auto finish_group = [&](int g, const f32x4(&v)[kE]) {
      int mat;
      const int r0 = group_row0(g, mat);
      float *logits = KQ_PH(ph, logits[mat]);
      const int nrows = (N - r0) < kRows ? (N - r0) : kRows;
#pragma unroll
      for (int j = 0; j < kE; ++j) {
        const int c = tid + j * kNth;
        const int row = c / kCR, m0 = 4 * (c % kCR);
        const int n = r0 + row;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + r;
          const bool ok = m < M && row < nrows;
          if (ok && logits) put(&logits[(int64_t)m * N + n], v[j][r]);
          if (a.verify) {
            unsigned long long best = ok ? argmax_key(v[j][r], (unsigned)n) : 0ull;
            if constexpr ((kCR & (kCR - 1)) == 0) {
              // max over the wave's 64 / kCR rows: the lanes with the same c % kCR
              best = lanes_max(best, 64, kCR);
              if (lane < kCR && m < M) atomicMax(&s_keys[m], best);
            } else {
              // three slices (12 chunks a row): lanes of one activation row
              // are not an xor group, so every lane goes to LDS on its own
              if (ok) atomicMax(&s_keys[m], best);
            }
          }
        }
      }
    };
    auto reduce_groups = [&](int ga, int gb, bool both) {
      const Contributors ca = contributors(ga);
      const Contributors cbb = contributors(both ? gb : ga);
      const int na = ca.pl - ca.pf + 1;
      const int nb = both ? cbb.pl - cbb.pf + 1 : 0;
      const int nmax = na > nb ? na : nb;
      f32x4 va[kE], vb[kE];
#pragma unroll
      for (int j = 0; j < kE; ++j) va[j] = vb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nmax; c0 += kC) {
        f32x4 pa[kE][kC], pb[kE][kC];
        load_partials(ca, c0, pa);
        if (both) load_partials(cbb, c0, pb);
        sum_partials(ca, c0, pa, va);
        if (both) sum_partials(cbb, c0, pb, vb);
      }
      finish_group(ga, va);
      if (both) finish_group(gb, vb);
    };

    if (have_first || last_partial) {
      if (MS == 1 && have_first) write_partial(0, acc_first);
      if (last_partial) write_partial(1, acc);
      // contributor counts of both groups (computed while the stores drain)
      int c_first = 0, c_last = 0;
      if (tid == 0) {
        c_first = owner(g_first * KB + KB - 1) - owner(g_first * KB) + 1;
        c_last = owner(g_last * KB + KB - 1) - owner(g_last * KB) + 1;
      }
      stores_done_barrier();
      if (tid == 0) {
        // both arrivals in flight at once; a group this workgroup has no
        // partial for gets an increment of 0
        unsigned *cnt_f = a.group_cnt + (int64_t)g_first * kCntStride;
        unsigned *cnt_l = a.group_cnt + (int64_t)g_last * kCntStride;
        const unsigned old_f = __hip_atomic_fetch_add(cnt_f, have_first ? 1u : 0u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        const unsigned old_l = __hip_atomic_fetch_add(cnt_l, last_partial ? 1u : 0u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        int flags = 0;
        if (have_first && old_f == (unsigned)(c_first - 1)) {
          __hip_atomic_store(cnt_f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          flags |= 1;
        }
        if (last_partial && old_l == (unsigned)(c_last - 1)) {
          __hip_atomic_store(cnt_l, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          flags |= 2;
        }
        s_flag = flags;
      }
      __syncthreads();
      const int flags = s_flag;
      if (flags == 3) {
        reduce_groups(g_first, g_last, true);
      } else if (flags) {
        reduce_groups(flags == 1 ? g_first : g_last, 0, false);
      }
    }


    if (!a.verify) return;
    __syncthreads();
    if (tid < kRS) st_dev(&a.wg_keys[(int64_t)p * kMaxTreeRows + tid], s_keys[tid]);
    stores_done_barrier();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = old == (unsigned)(P - 1);
    }
    __syncthreads();
    if (!s_flag) return;
    if (tid < kRS) s_keys[tid] = 0ull;
    __syncthreads();
    {
      const int m = tid % kRS;
      if (m < M) {
        unsigned long long best = 0ull;
        for (int q = tid / kRS; q < P; q += kNth / kRS) {
          const unsigned long long key = ld_dev(&a.wg_keys[(int64_t)q * kMaxTreeRows + m]);
          best = key > best ? key : best;
        }
        atomicMax(&s_keys[m], best);
      }
    }
    __syncthreads();
    const int MT = M;
    if (tid < M) {
      const int am = (int)(0xFFFFFFFFu - (unsigned)(s_keys[tid] & 0xFFFFFFFFull));
      s_am[tid] = am;
      if (tid >= a.argmax_from) a.argmax_out[tid - a.argmax_from] = am;
    }
    __syncthreads();
    if (a.accept_out && a.tree) {
      // Token tree: wave 0 walks from the root; lane j holds node j. Each
      // move goes to a higher node index (parents precede children), so the
      // walk ends within MT - 1 moves.
      if (tid < 64) {
        const int j = lane;
        const int par = j < MT ? a.parent[j] : -1;
        const int tok = j < MT ? a.draft[j] : -1;
        int cur = 0, n = 0;
        while (true) {
          const bool match = j >= 1 && j < MT && par == cur && tok == s_am[cur];
          const unsigned long long bal = __ballot(match);
          if (!bal) break;
          const int nxt = __ffsll((long long)bal) - 1;
          if (lane == 0 && a.path_out) a.path_out[n] = nxt;
          ++n;
          cur = nxt;
        }
        if (lane == 0) {
          a.accept_out[0] = n;
          a.accept_out[1] = s_am[cur];
        }
      }
    }
    if (tid == 0) {
      if (a.head_out) a.head_out[0] = s_am[0];
      if (a.accept_out && !a.tree) {
        // device drafts are only compared, never used as an index, so a
        // token outside [0, n) is a mismatch
        int i = 0;
        while (i < a.k_draft && (a.draft_dev ? a.draft_dev[i] : a.draft[i]) == s_am[i]) ++i;
        a.accept_out[0] = i;
        a.accept_out[1] = s_am[i];
      }
      __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

#undef KQ_PH

// ---------------------------------------------------------------------------
// Chain launches with specialised waves (kq_chain_kernel). A workgroup has
// kCwW compute waves (one 16-row tile each: row groups of 128 rows, units
// as in kq_gemv_kernel) and kCwP producer waves:
//  * compute waves only load weights and compute: kCwD register sets, the
//    weights of a unit issued kCwD - 1 units before it is computed, in one
//    stream that runs through the phases (a phase's last units already
//    carry the next phase's first weights, which do not depend on the
//    barrier). Their memory counter holds nothing but weight loads, so
//    waiting for one unit's weights never waits for anything younger: the
//    reason this prefetch can run deeper than kq_gemv_kernel's, where the
//    activation loads and the stores share the counter;
//  * producer waves copy each unit's staged activations into the LDS ring
//    one barrier interval ahead (direct-to-LDS buffer loads, no register
//    staging), and do every global store: the
//    results the compute waves hand over through LDS (a finished row group's
//    logits, a later contributor's partial sums), the pull reduction of a
//    split row group, and the grid barrier between phases.
// A phase's units, its row-group arithmetic and its summation orders are
// those of kq_gemv_kernel, so the results are bitwise equal to it.
// ---------------------------------------------------------------------------

constexpr int kCwW = 8;                                // compute waves
constexpr int kCwT = 1;                                // 16-row tiles per compute wave
constexpr int kCwP = 4;                                // producer waves
constexpr int kCwD = 4;                                // weight register sets per compute wave
constexpr int kCwBI = 4;                               // most units between workgroup barriers
constexpr int kCwRows = 16 * kCwW * kCwT;              // rows per row group (128)
constexpr int kCwPT = 64 * kCwP;                       // producer threads
constexpr int kCwXc = (int)(kStageBytes / 16);         // 16-byte chunks of a staged block (1,060)
constexpr int kCwXj = (kCwXc + kCwPT - 1) / kCwPT;     // LDS copy instructions per producer wave and block (5)
constexpr int kCwChunks = kCwRows * kMaxRows / 4;      // 16-byte chunks of a row group's result (512)
constexpr int kCwE = kCwChunks / kCwPT;                // of them per producer thread (2)
constexpr int kCwC = 8;                                // contributors' partials in flight in a pull
static_assert(kCwE * kCwPT == kCwChunks, "result chunks split evenly over the producer threads");
static_assert((kCwBI & (kCwBI - 1)) == 0, "barrier interval a power of two");
static_assert(kCwP == 4 && kCwXc <= 64 * 4 * kCwXj, "4 producer waves cover a block in kCwXj KiB runs each");
static_assert(kCwRows == kChainRows, "row groups of the chain geometry");

// One unit of T 16-row tiles of Q4_K weights: per tile, block d, dmin, the
// 6-bit scales and mins unpacked in registers, the 4-bit quants times their
// scale as exact fp16 B operands, contracted with the staged activations xb
// (hi and lo halves into one fp32 sum; every A operand read from LDS feeds
// all T tiles), the min term as one 16x16x16 MFMA; acc[t] gains
// 2^-e (d C - dmin C_m). Per tile, the same operations in the same order as
// the Q4_K path of kq_gemv_kernel.
template <int T>
__device__ __forceinline__ void q4_unit(const WTile (&cur)[T], const uint8_t *xb, int lane, int kg, unsigned sel_sc,
                                        unsigned mask_lo, unsigned mask_hi, f32x4 (&acc)[T]) {
  const half2v neg1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const half2v lo_pair = {(_Float16)1.0f, (_Float16)-1024.0f};
  const half2v hi_pair = {(_Float16)0.0625f, (_Float16)-64.0f};
  float d[T], dmin[T];
  half2v k00[T], k01[T], k10[T], k11[T];
  half4 bm[T];
  f32x4 cq[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const u32x4 h = cur[t].hdr;
    d[t] = h2f_lo(h.x);
    dmin[t] = h2f_hi(h.x);
    const unsigned sc03 = h.y & 0x3F3F3F3Fu;
    const unsigned sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const half2v s0 = as_h2(__builtin_amdgcn_perm(sc03, 0x64646464u, sel_sc)) + neg1024;
    const half2v s1 = as_h2(__builtin_amdgcn_perm(sc47, 0x64646464u, sel_sc)) + neg1024;
    k00[t] = half2v{s0[0], s0[0]} * lo_pair;
    k01[t] = half2v{s0[1], s0[1]} * hi_pair;
    k10[t] = half2v{s1[0], s1[0]} * lo_pair;
    k11[t] = half2v{s1[1], s1[1]} * hi_pair;
    const unsigned m03 = h.z & 0x3F3F3F3Fu;
    const unsigned m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const unsigned msrc = (kg & 1) ? m47 : m03;
    const half2v p0 = as_h2(__builtin_amdgcn_perm(msrc, 0x64646464u, 0x00060004u)) + neg1024;
    const half2v p1 = as_h2(__builtin_amdgcn_perm(msrc, 0x64646464u, 0x00070005u)) + neg1024;
    bm[t] = half4{p0[0], p0[1], p1[0], p1[1]};
    cq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // A operands (x hi and lo of k-step s) read from LDS two k-steps before
  // their MFMAs, in three rotating register pairs; the scheduling fences
  // keep each read ahead of the work it should overlap with
  constexpr int kAP = 2;
  half8 ahi_r[kAP + 1], alo_r[kAP + 1];
  const uint8_t *xa = xb + lane * 16;
#pragma unroll
  for (int s = 0; s < kAP; ++s) {
    ahi_r[s] = *(const half8 *)(xa + (s * 2 + 0) * 1024);
    alo_r[s] = *(const half8 *)(xa + (s * 2 + 1) * 1024);
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + kAP < 8) {
      ahi_r[(s + kAP) % (kAP + 1)] = *(const half8 *)(xa + ((s + kAP) * 2 + 0) * 1024);
      alo_r[(s + kAP) % (kAP + 1)] = *(const half8 *)(xa + ((s + kAP) * 2 + 1) * 1024);
    }
    __builtin_amdgcn_sched_barrier(0);
    const half8 ahi = ahi_r[s % (kAP + 1)];
    const half8 alo = alo_r[s % (kAP + 1)];
    const bool hi = (s & 2) != 0;
    const unsigned mask = hi ? mask_hi : mask_lo;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const u32x4 qq = s < 4 ? cur[t].q0 : cur[t].q1;
      const unsigned da = (s & 1) ? qq.z : qq.x;
      const unsigned db = (s & 1) ? qq.w : qq.y;
      const half2v kk = s < 4 ? (hi ? k01[t] : k00[t]) : (hi ? k11[t] : k10[t]);
      const half2v v0 = fma_bcast(as_h2((da & mask) | 0x64006400u), kk);
      const half2v v1 = fma_bcast(as_h2(((da >> 8) & mask) | 0x64006400u), kk);
      const half2v v2 = fma_bcast(as_h2((db & mask) | 0x64006400u), kk);
      const half2v v3 = fma_bcast(as_h2(((db >> 8) & mask) | 0x64006400u), kk);
      const half8 bw8 = make_h8(as_u(v0), as_u(v1), as_u(v2), as_u(v3));
      cq[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bw8, cq[t], 0, 0, 0);
      cq[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bw8, cq[t], 0, 0, 0);
    }
  }
  const half4 as4 = *(const half4 *)(xb + kXsbOffset + lane * 8);
  const f32x4 xinv = *(const f32x4 *)(xb + kXiOffset + 16 * kg);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const f32x4 c2 = __builtin_amdgcn_mfma_f32_16x16x16f16(as4, bm[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] += xinv[r] * (d[t] * cq[t][r] - dmin[t] * c2[r]);
  }
}

// Barrier of the producer waves alone (the compute waves are meanwhile at a
// workgroup barrier of their own, which an s_barrier here would complete):
// an LDS arrival count. Bounded like every wait; false after a time-out.
__device__ __forceinline__ bool producer_bar(unsigned *cnt, unsigned &target) {
  target += kCwP;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while ((int)(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) - target) < 0) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return true;
}

#define KQ_CPH(I_, f) (SINGLE ? a.ph.f : ((const __attribute__((address_space(4))) Phase *)a.chain)[(I_)].f)

// ROWS: Q4_K weights in llama.cpp rows (else tiled), as for kq_gemv_kernel.
// SINGLE: a single launch's one phase (a.ph, no table, no grid barrier);
// split row groups are then combined as kq_gemv_kernel combines them, by the
// last contributor to arrive, so no workgroup ever waits for another and the
// launch needs no co-residency.
template <bool ROWS, bool SINGLE>
__global__ __launch_bounds__(64 * (kCwW + kCwP), 1) void kq_chain_kernel(GemvLaunch a) {
  // LDS: the activation ring (two halves of up to kCwBI staged blocks: the
  // compute waves read one half while the producers fill the other; after
  // a phase's last unit the unused half takes the final hand-over), two
  // hand-over slots for results finished inside a run, and control words.
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2 * kCwBI][kStageBytes];
  __shared__ __attribute__((aligned(16))) float s_hand[2][kCwRows * kMaxRows];
  __shared__ int s_hdesc[2];   // hand-over in slot i: group * 4 + kind
  __shared__ int s_htag[2];    // ... written in the launch's interval s_htag[i]
  __shared__ int s_fdesc;      // the final hand-over of a phase
  __shared__ unsigned s_pbar;  // producer barrier count
  __shared__ unsigned s_bad;   // producer broadcast words: a partial never arrived,
  __shared__ unsigned s_last;  // this arrival completed the grid barrier (single launches: the groups it reduces),
  __shared__ unsigned s_ok;    // the barrier wait ended with a release
  __shared__ int s_abort;      // set by the producers when a wait gave up
  __shared__ unsigned long long s_epoch;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kg = lane >> 4;
  const int ln = lane & 15;
  const int M = a.m;
  const int P = gridDim.x;
  const int p = blockIdx.x;
  const int n_ph = SINGLE ? 1 : a.n_phases;
  constexpr bool tiled = !ROWS;
  // hand-over kinds: a row group finished here (its logits), a later
  // contributor's partial (to its slot 0, pulled by the group's first
  // contributor), a group this workgroup reduces (pull, then logits)
  constexpr int kKindDone = 0, kKindPartial = 1, kKindReduce = 2;

  auto run_start = [&](int U) -> int {
    const int b = U / P, r = U % P;
    return p * b + (p < r ? p : r);
  };
  auto run_len = [&](int U) -> int { return U / P + (p < U % P ? 1 : 0); };
  // log2 of the units between barriers: kCwBI, fewer (a power of two) for
  // rows of fewer blocks, so that at most one row group ends inside an
  // interval and two hand-over slots suffice
  auto interval_log2 = [&](int KB) -> int { return KB >= 4 ? 2 : KB >= 2 ? 1 : 0; };
  // LDS buffer of unit i of a phase (interval 2^lb)
  auto ring_buf = [&](int i, int lb) -> int { return ((i >> lb) & 1) * kCwBI + (i & ((1 << lb) - 1)); };
  // row of tile t of a compute wave within its row group
  auto tile_row = [&](int t) -> int { return (t * kCwW + wave) * 16 + ln; };

  if (tid == 0) {
    s_last = 0u;
    s_htag[0] = s_htag[1] = -1;
    s_pbar = 0u;
    s_bad = 0u;
    s_abort = 0;
    if (!SINGLE) {
      s_epoch = (unsigned long long)__hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) << 32;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the epoch is read before any arrival
    }
  }

  if (wave < kCwW) {
    // ------------------------------------------------------------ compute
    const unsigned mask_lo = in_vgpr(0x000F000Fu);
    const unsigned mask_hi = in_vgpr(0x00F000F0u);
    const unsigned sel_sc = (kg >> 1) ? 0x00070006u : 0x00050004u;
    // the weight stream (its own copy of its phase's geometry)
    int wp = 0, uw = 0, uw_last = 0, gw = 0, bw = 0;
    int cw_n = 1, cw_rb = 0, cw_nt = 1, cw_kb = 1, cw_nwg = 1;
    unsigned boff = 0, bstride = 0;
    __amdgpu_buffer_rsrc_t w_rsrc;
    unsigned voff[kCwT][3], soff[kCwT];
    auto set_rowp = [&]() {
      const int mat = gw / cw_nwg;
      const int r0 = (gw - mat * cw_nwg) * kCwRows;
      w_rsrc = dev_rsrc(KQ_CPH(wp, w[mat]));
#pragma unroll
      for (int t = 0; t < kCwT; ++t) {
        if (tiled) {
          int ti = (r0 + (t * kCwW + wave) * 16) / 16;
          ti = ti < cw_nt ? ti : cw_nt - 1;
          soff[t] = (unsigned)ti * (unsigned)kTileBlockBytes;
          voff[t][0] = 16u * ln;
          voff[t][1] = (unsigned)kTileQ0 + 16u * lane;
          voff[t][2] = (unsigned)kTileQ1 + 16u * lane;
        } else {
          const int row = r0 + tile_row(t);
          const unsigned rb = (unsigned)(row < cw_n ? row : cw_n - 1) * (unsigned)cw_rb;
          soff[t] = 0u;
          voff[t][0] = rb;
          voff[t][1] = rb + 16u + 16u * kg;
          voff[t][2] = rb + 80u + 16u * kg;
        }
      }
    };
    auto begin_w = [&](int ph) {
      wp = ph;
      const int U = KQ_CPH(ph, units);
      cw_n = KQ_CPH(ph, n);
      cw_rb = KQ_CPH(ph, row_bytes);
      cw_nt = KQ_CPH(ph, n_tiles);
      cw_kb = KQ_CPH(ph, kb);
      cw_nwg = KQ_CPH(ph, n_wg_per);
      bstride = tiled ? (unsigned)cw_nt * (unsigned)kTileBlockBytes : (unsigned)kBlockBytes;
      uw = run_start(U);
      uw_last = uw + run_len(U) - 1;
      gw = uw / cw_kb;
      bw = uw % cw_kb;
      boff = (unsigned)bw * bstride;
      set_rowp();
    };
    // issue the loads of the stream's next unit and advance (into the next
    // phase after this one's last unit; the last phase's last unit repeats)
    auto load_w = [&](WTile (&w)[kCwT]) {
#pragma unroll
      for (int t = 0; t < kCwT; ++t) {
        load_q4_tile(w[t], w_rsrc, voff[t], soff[t] + boff, tiled);
      }
      if (uw < uw_last) {
        ++uw;
        boff += bstride;
        if (++bw == cw_kb) {
          bw = 0;
          boff = 0u;
          ++gw;
          set_rowp();
        }
      } else if (wp + 1 < n_ph) {
        begin_w(wp + 1);
      }
    };

    // One loop over the launch's steps (every unit of every phase in order),
    // unrolled kCwD times so that the register set of each step is static.
    // Each step issues the loads of the stream's unit kCwD - 1 steps ahead
    // unconditionally (past the last phase the last unit repeats), so the
    // memory counter waits are static too; the phase tail (hand-over,
    // barriers) is a branch inside the step of a phase's last unit.
    WTile wr[kCwD][kCwT];
    int S = 0;  // this workgroup's units over all phases
    for (int q = 0; q < n_ph; ++q) S += run_len(KQ_CPH(q, units));
    begin_w(0);
#pragma unroll
    for (int d = 0; d < kCwD - 1; ++d) load_w(wr[d]);

    // phase state: ph; KB, nu, lb of the phase; gc, bc, seg0 the current
    // row group, block and segment start; i the unit, ib its place in its
    // barrier interval, kint the interval; gint the launch's intervals
    // before this phase (hand-over tags)
    int ph = 0, gint = 0, KB = 1, nu = 1, lb = 0, gc = 0, bc = 0, seg0 = 0, i = 0, ib = 0, kint = 0;
    auto enter = [&](int q) {
      KB = KQ_CPH(q, kb);
      const int U = KQ_CPH(q, units);
      const int u0 = run_start(U);
      nu = run_len(U);
      lb = interval_log2(KB);
      gc = u0 / KB;
      bc = u0 - gc * KB;
      seg0 = bc;
      i = ib = kint = 0;
    };
    enter(0);
    f32x4 acc[kCwT];
#pragma unroll
    for (int t = 0; t < kCwT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // the first phase's first activations are in the ring
    if (s_abort) return;
    for (int s0 = 0; s0 < S; s0 += kCwD) {
#pragma unroll
      for (int j = 0; j < kCwD; ++j) {
        // the two compute waves of a SIMD take turns at the higher issue
        // priority, one step each, so that one of them runs ahead and their
        // memory waits and MFMA chains do not line up
        if ((wave >> 2) == (j & 1))
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
        load_w(wr[(j + kCwD - 1) % kCwD]);
        __builtin_amdgcn_sched_barrier(0);
        if (s0 + j < S) {
          q4_unit<kCwT>(wr[j], s_x[((kint & 1) * kCwBI) + ib], lane, kg, sel_sc, mask_lo, mask_hi, acc);
          // end of a row group's segment: hand the result to the producers
          if (bc == KB - 1 || i == nu - 1) {
            const int kind = (seg0 == 0 && bc == KB - 1) ? kKindDone : seg0 > 0 ? kKindPartial : kKindReduce;
            const int gi = gint + kint;  // the launch's interval of this unit
            float *dst = i == nu - 1 ? (float *)s_x[((kint + 1) & 1) * kCwBI] : s_hand[gi & 1];
#pragma unroll
            for (int t = 0; t < kCwT; ++t) {
              *(f32x4 *)(dst + tile_row(t) * kMaxRows + 4 * kg) = acc[t];
              acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (tid == 0) {
              if (i == nu - 1) {
                s_fdesc = gc * 4 + kind;
              } else {
                s_hdesc[gi & 1] = gc * 4 + kind;
                s_htag[gi & 1] = gi;
              }
            }
            seg0 = 0;
          }
          if (++bc == KB) {
            bc = 0;
            ++gc;
          }
          if (i == nu - 1) {
            // phase tail: the producers store, reduce and pass the grid
            // barrier; the weights of the next phase stay in flight
            gint += kint + 1;
            __syncthreads();  // the phase's results are handed over
            if (ph + 1 < n_ph) {
              enter(++ph);
              __syncthreads();  // the next phase's first activations are in the ring
              if (s_abort) {
                __builtin_amdgcn_s_waitcnt(0x0F70);
                return;
              }
            }
          } else {
            ++i;
            if (++ib == (1 << lb)) {
              ib = 0;
              ++kint;
              __syncthreads();  // the next interval's activations are in
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the repeated last loads
    return;
  }

  // -------------------------------------------------------------- producers
  const int pt = tid - 64 * kCwW;
  unsigned pbar_target = 0;
  const __amdgpu_buffer_rsrc_t part_rsrc = dev_rsrc(a.partials);
  // Activations of units i .. i_end - 1 (< i + kCwBI) of phase ph into the
  // ring (their blocks' staged records, copied linearly): all loads first,
  // then `between` (hand-over stores overlap the loads), then the LDS writes.
  auto move_x = [&](int ph, int i, int i_end, int lb, auto between) {
    const int KB = KQ_CPH(ph, kb);
    const int u0 = run_start(KQ_CPH(ph, units));
    const __amdgpu_buffer_rsrc_t x_rsrc = dev_rsrc(KQ_CPH(ph, staged));
    // buffer_load_dwordx4 ... lds: every lane's 16 bytes go straight to LDS
    // at the wave's base + 16 x lane, so instruction j of producer wave pw
    // copies chunks 64 (4 j + pw) .. + 63 of a block (one contiguous KiB)
    const int pw = __builtin_amdgcn_readfirstlane(pt >> 6), ln = pt & 63;
#pragma unroll
    for (int q = 0; q < kCwBI; ++q) {
      if (i + q < i_end) {
        const unsigned src = (unsigned)((u0 + i + q) % KB) * (unsigned)kStageBytes;
        uint8_t *dst = s_x[ring_buf(i + q, lb)];
#pragma unroll
        for (int j = 0; j < kCwXj; ++j) {
          const int cb = 64 * (4 * j + pw);
          if (cb < kCwXc && cb + ln < kCwXc)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (__attribute__((address_space(3))) void *)(dst + cb * 16),
                                                     16, (unsigned)(cb + ln) * 16u, src, 0, 0);
        }
      }
    }
    between();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the blocks are in LDS
  };
  // logits of row group g of phase ph from a result ([row][16] fp32, the
  // thread's chunks pt + j kCwPT)
  auto store_logits = [&](int ph, int g, const f32x4 (&v)[kCwE]) {
    const int N = KQ_CPH(ph, n);
    const int nwg = KQ_CPH(ph, n_wg_per);
    const int mat = g / nwg;
    const int r0 = (g - mat * nwg) * kCwRows;
    float *logits = KQ_CPH(ph, logits[mat]);
#pragma unroll
    for (int j = 0; j < kCwE; ++j) {
      const int c = pt + j * kCwPT;
      const int row = c >> 2, m0 = 4 * (c & 3);
      if (r0 + row < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (m0 + r < M) st_dev(&logits[(int64_t)(m0 + r) * N + r0 + row], v[j][r]);
      }
    }
  };
  auto load_hand = [&](const float *src, f32x4 (&v)[kCwE]) {
#pragma unroll
    for (int j = 0; j < kCwE; ++j) v[j] = *(const f32x4 *)(src + 4 * (pt + j * kCwPT));
  };
  auto slot0 = [&](int q) -> unsigned { return (unsigned)(q * 2 * kMaxRows * kCwRows) * 4u; };
  // a hand-over finished inside a run: logits, or this workgroup's partial
  auto store_hand = [&](int ph, int desc, const float *src) {
    f32x4 v[kCwE];
    load_hand(src, v);
    if ((desc & 3) == kKindDone) {
      store_logits(ph, desc >> 2, v);
    } else {
#pragma unroll
      for (int j = 0; j < kCwE; ++j) st_dev16(part_rsrc, slot0(p) + (unsigned)(pt + j * kCwPT) * 16u, v[j]);
    }
  };
  // every producer wave ends here when a wait gave up: the compute waves
  // leave at their next phase barrier
  auto abort_all = [&]() {
    if (pt == 0) {
      __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_abort = 1;
    }
    __syncthreads();
  };

  {
    const int nu = run_len(KQ_CPH(0, units));
    const int lb = interval_log2(KQ_CPH(0, kb));
    move_x(0, 0, nu < (1 << lb) ? nu : (1 << lb), lb, [] {});
  }
  int gint = 0;  // barrier intervals of the earlier phases (hand-over tags)
  for (int ph = 0; ph < n_ph; ++ph) {
    const int KB = KQ_CPH(ph, kb);
    const int U = KQ_CPH(ph, units);
    const int nu = run_len(U);
    const int lb = interval_log2(KB);
    const int bi = 1 << lb;
    const int n_int = (nu + bi - 1) >> lb;
    // a hand-over written in the launch's interval gi, if any (slots are
    // tagged with the interval that wrote them, so nothing is cleared)
    auto hand_of = [&](int gi) {
      if (gi >= 0 && s_htag[gi & 1] == gi) store_hand(ph, s_hdesc[gi & 1], s_hand[gi & 1]);
    };
    __syncthreads();  // the phase starts
    for (int k = 0; k < n_int; ++k) {
      // the activations of interval k + 1; meanwhile the hand-over of
      // interval k - 1 (published by the barrier that ended it)
      const int i1 = (k + 1) * bi;
      move_x(ph, i1, nu < i1 + bi ? nu : i1 + bi, lb, [&] {
        if (k > 0) hand_of(gint + k - 1);
      });
      __syncthreads();  // interval k's units done; interval k + 1's activations in
    }
    // ---- phase tail (producer waves only; the compute waves wait at the
    // next phase's barrier)
    hand_of(gint + n_int - 1);
    gint += n_int;
    const int fdesc = s_fdesc;
    const float *fin = (const float *)s_x[(n_int & 1) * kCwBI];
    if constexpr (SINGLE) {
      // A single launch combines split row groups as kq_gemv_kernel does:
      // this workgroup's partial of its first group (when that group is not
      // complete here) is in slot 0, its partial of a later last group in
      // slot 1; once they are written, it arrives at each group's count, and
      // the last contributor to arrive sums all of them in workgroup order.
      const int base = U / P, rem = U % P;
      const int big = rem * (base + 1);
      auto owner = [&](int u) -> int { return u < big ? u / (base + 1) : rem + (u - big) / base; };
      auto start_of = [&](int q) -> int { return q * base + (q < rem ? q : rem); };
      const int u0 = start_of(p), u_last = u0 + nu - 1;
      const int g_first = u0 / KB, g_last = u_last / KB;
      const int have_first = (u0 % KB != 0) || (u_last < g_first * KB + KB - 1);
      const int last_partial = (g_last != g_first) && (u_last % KB != KB - 1);
      constexpr unsigned kSlotBytes = (unsigned)(kMaxRows * kCwRows) * 4u;
      if ((fdesc & 3) == kKindReduce) {
        // the final segment opened its group: slot 1 unless it is also the
        // first segment (then its group is the first group: slot 0)
        f32x4 v[kCwE];
        load_hand(fin, v);
        const unsigned slot = (fdesc >> 2) != g_first ? kSlotBytes : 0u;
#pragma unroll
        for (int j = 0; j < kCwE; ++j) st_dev16(part_rsrc, slot0(p) + slot + (unsigned)(pt + j * kCwPT) * 16u, v[j]);
      } else {
        store_hand(ph, fdesc, fin);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
      if (!producer_bar(&s_pbar, pbar_target)) {
        abort_all();
        return;
      }
      if (pt == 0) {
        unsigned flags = 0u;
        if (have_first || last_partial) {
          unsigned *cnt_f = a.group_cnt + (int64_t)g_first * kCntStride;
          unsigned *cnt_l = a.group_cnt + (int64_t)g_last * kCntStride;
          const unsigned old_f =
              __hip_atomic_fetch_add(cnt_f, have_first ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const unsigned old_l =
              __hip_atomic_fetch_add(cnt_l, last_partial ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int c_first = owner(g_first * KB + KB - 1) - owner(g_first * KB) + 1;
          const int c_last = owner(g_last * KB + KB - 1) - owner(g_last * KB) + 1;
          if (have_first && old_f == (unsigned)(c_first - 1)) {
            __hip_atomic_store(cnt_f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            flags |= 1u;
          }
          if (last_partial && old_l == (unsigned)(c_last - 1)) {
            __hip_atomic_store(cnt_l, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            flags |= 2u;
          }
        }
        s_last = flags;
      }
      if (!producer_bar(&s_pbar, pbar_target)) {
        abort_all();
        return;
      }
      const unsigned flags = s_last;
      // sum group g over its contributors pf .. pl (pf's partial in its
      // slot 1 when its run starts before g, the others' in slot 0), the
      // loads of kCwC contributors in flight together
      auto reduce = [&](int g) {
        const int pf = owner(g * KB), pl = owner(g * KB + KB - 1);
        const unsigned pf_slot = start_of(pf) < g * KB ? kSlotBytes : 0u;
        f32x4 v[kCwE];
#pragma unroll
        for (int j = 0; j < kCwE; ++j) v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 <= pl - pf; c0 += kCwC) {
          f32x4 pv[kCwE][kCwC];
#pragma unroll
          for (int c = 0; c < kCwC; ++c) {
            const int q = pf + c0 + c <= pl ? pf + c0 + c : pl;
            const unsigned src = slot0(q) + (q == pf ? pf_slot : 0u);
#pragma unroll
            for (int j = 0; j < kCwE; ++j) pv[j][c] = ld_dev16(part_rsrc, src + (unsigned)(pt + j * kCwPT) * 16u);
          }
#pragma unroll
          for (int c = 0; c < kCwC; ++c)
#pragma unroll
            for (int j = 0; j < kCwE; ++j)
              if (pf + c0 + c <= pl) v[j] = c0 + c == 0 ? pv[j][c] : v[j] + pv[j][c];
        }
        store_logits(ph, g, v);
      };
      if (flags & 1u) reduce(g_first);
      if (flags & 2u) reduce(g_last);
      continue;  // one phase: the loop ends here
    }
    int bad = 0;
    if ((fdesc & 3) == kKindReduce) {
      // pull: sum the later contributors' partials of group g in workgroup
      // order after this workgroup's own (the group's first part)
      const int g = fdesc >> 2;
      const int big = (U % P) * (U / P + 1);
      auto owner = [&](int u) -> int { return u < big ? u / (U / P + 1) : U % P + (u - big) / (U / P); };
      const int plg = owner(g * KB + KB - 1);
      f32x4 v[kCwE];
      load_hand(fin, v);
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      for (int c0 = 1; c0 <= plg - p; c0 += kCwC) {
        f32x4 pv[kCwE][kCwC];
#pragma unroll
        for (int c = 0; c < kCwC; ++c) {
          const int q = p + c0 + c <= plg ? p + c0 + c : plg;
#pragma unroll
          for (int j = 0; j < kCwE; ++j) pv[j][c] = ld_dev16(part_rsrc, slot0(q) + (unsigned)(pt + j * kCwPT) * 16u);
        }
#pragma unroll
        for (int c = 0; c < kCwC; ++c) {
          if (p + c0 + c > plg) continue;
#pragma unroll
          for (int j = 0; j < kCwE; ++j) {
            while (true) {  // not yet written: poll (bounded)
              const u32x4 w = __builtin_bit_cast(u32x4, pv[j][c]);
              if (w.x != 0xFFFFFFFFu && w.y != 0xFFFFFFFFu && w.z != 0xFFFFFFFFu && w.w != 0xFFFFFFFFu) break;
              if (bad || __builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
                bad = 1;
                break;
              }
              __builtin_amdgcn_s_sleep(1);
              pv[j][c] = ld_dev16(part_rsrc, slot0(p + c0 + c) + (unsigned)(pt + j * kCwPT) * 16u);
            }
            v[j] = v[j] + pv[j][c];
          }
        }
      }
      if (!bad) {
        store_logits(ph, g, v);
        // consumed slots back to the sentinel before this workgroup arrives
        const f32x4 sentinel =
            __builtin_bit_cast(f32x4, u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
        for (int q = p + 1; q <= plg; ++q)
#pragma unroll
          for (int j = 0; j < kCwE; ++j) st_dev16(part_rsrc, slot0(q) + (unsigned)(pt + j * kCwPT) * 16u, sentinel);
      }
    } else {
      store_hand(ph, fdesc, fin);
    }
    if (bad) __hip_atomic_fetch_or(&s_bad, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
    if (!producer_bar(&s_pbar, pbar_target) || s_bad) {
      abort_all();
      return;  // a partial never arrived (or the producers lost each other)
    }
    // grid barrier: arrive; the arrival that completes the count releases
    // every other workgroup through its own flag (see kq_gemv_kernel)
    const unsigned target = (unsigned)(ph + 1) * (unsigned)P;
    if (ph + 1 < n_ph) {
      if (pt == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old + 1 == target ? 1u : 0u;
      }
      if (!producer_bar(&s_pbar, pbar_target)) {
        abort_all();
        return;
      }
      const unsigned long long want = s_epoch | (unsigned long long)(ph + 1);
      if (s_last) {
        for (int q = pt; q < P; q += kCwPT)
          if (q != p) st_dev(a.flags + (int64_t)q * kFlagStride, want);
        if (pt == 0) s_ok = 1u;
      } else if (pt == 0) {
        s_ok = spin_flag(a.flags + (int64_t)p * kFlagStride, want, a.err) ? 1u : 0u;
      }
      if (pt == 0) s_bad = 0u;  // every producer read it before the last barrier
      if (!producer_bar(&s_pbar, pbar_target) || !s_ok) {
        abort_all();
        return;  // the barrier wait gave up
      }
      // the next phase's first activations, read only now
      const int nu1 = run_len(KQ_CPH(ph + 1, units));
      const int lb1 = interval_log2(KQ_CPH(ph + 1, kb));
      move_x(ph + 1, 0, nu1 < (1 << lb1) ? nu1 : (1 << lb1), lb1, [] {});
    } else if (pt == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == target) {
        __hip_atomic_store(a.bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(a.epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

#undef KQ_CPH

// ---------------------------------------------------------------------------
// Tiled layout. Record (b, t) = block b of 16-row tile t is 2,304 bytes at
// (b * tiles + t) * 2,304: the 16 headers (row order), then bytes [16kg,
// 16kg + 16) of the quants of row ln at 256 + 16 (16 kg + ln), then bytes
// [64 + 16kg, 80 + 16kg) at 1,280 + 16 (16 kg + ln). Rows past n are zero.
// One thread per 16-byte output chunk.
__global__ __launch_bounds__(256) void kq_tile_kernel(const uint8_t *__restrict__ w, int64_t n,
                                                      int64_t kb, int64_t n_tiles,
                                                      uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = kb * n_tiles * 144;
  if (idx >= total) return;
  const int c = (int)(idx % 144);
  const int64_t tb = idx / 144;
  const int64_t ti = tb % n_tiles;
  const int64_t b = tb / n_tiles;
  int ln, chunk;
  if (c < 16) {
    ln = c;
    chunk = 0;
  } else if (c < 80) {
    ln = (c - 16) & 15;
    chunk = 1 + ((c - 16) >> 4);
  } else {
    ln = (c - 80) & 15;
    chunk = 5 + ((c - 80) >> 4);
  }
  const int64_t row = ti * 16 + ln;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < n) v = ld16(w + (row * kb + b) * kBlockBytes + chunk * 16);
  *(u32x4 *)(out + idx * 16) = v;
}

// ---------------------------------------------------------------------------
// Q5_K and Q6_K tiled records (layouts in kq.h). One thread per (block,
// tile, row): it reads the row's block and writes every byte that row owns
// in the record (its header or scale words, the 16-byte quant chunks of its
// four lanes, their high-bit words, its d). Lane group g of the row holds,
// in k-step s at byte p of its 8 bytes, block column lane_col(g, s, p): the
// column order the Q4_K records and the staged activations use.
__device__ __forceinline__ int lane_col(int g, int s, int p) {
  const int gg = (s < 4 ? 0 : 2) + (g >> 1), h = (s >> 1) & 1, l = 16 * (g & 1) + 8 * (s & 1) + p;
  return 64 * gg + 32 * h + l;
}

template <int FMT>
__global__ __launch_bounds__(256) void kq_tile_kq_kernel(const uint8_t *__restrict__ w, int64_t n, int64_t kb,
                                                         int64_t n_tiles, uint8_t *__restrict__ out) {
  constexpr int BB = (int)fmt_block_bytes(FMT);
  // the bytes of a pair of weights in an unpacked word: (0,2), (1,3), (4,6), (5,7)
  constexpr int kPair[4][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}};
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= kb * n_tiles * 16) return;
  const int r = (int)(idx & 15);
  const int64_t tb = idx >> 4, ti = tb % n_tiles, b = tb / n_tiles;
  const int64_t row = ti * 16 + r;
  const bool live = row < n;
  const uint8_t *src = w + (live ? (row * kb + b) * BB : 0);
  uint8_t *rec = out + (b * n_tiles + ti) * 16 * BB;
  auto byte = [&](int i) -> unsigned { return live ? (unsigned)src[i] : 0u; };
  if constexpr (FMT == kFmtQ5) {
    // d, dmin, 12 scale bytes | qh[32] at 16 | qs[128] at 48
    for (int i = 0; i < 16; ++i) rec[16 * r + i] = (uint8_t)byte(i);
    for (int g = 0; g < 4; ++g) {
      const int ln = 16 * g + r;
      for (int j = 0; j < 16; ++j) {
        rec[kTileQ0 + 16 * ln + j] = (uint8_t)byte(48 + 16 * g + j);
        rec[kTileQ1 + 16 * ln + j] = (uint8_t)byte(48 + 64 + 16 * g + j);
      }
      unsigned hw[2] = {0u, 0u};
      for (int s = 0; s < 8; ++s)
        for (int q = 0; q < 4; ++q)
          for (int e = 0; e < 2; ++e) {
            const int col = lane_col(g, s, kPair[q][e]);
            const unsigned bit = (byte(16 + col % 32) >> (col / 32)) & 1u;
            hw[s >> 2] |= bit << (4 * (s & 3) + q + 16 * e);
          }
      *(unsigned *)(rec + kTileQH + 8 * ln) = hw[0];
      *(unsigned *)(rec + kTileQH + 8 * ln + 4) = hw[1];
    }
  } else {
    // ql[128] | qh[64] at 128 | 16 signed scales at 192 | fp16 d at 208
    auto low4 = [&](int i) -> unsigned {
      const int h = i >> 7, c = (i & 127) >> 5, l = i & 31;
      const unsigned v = byte(64 * h + l + 32 * (c & 1));
      return c < 2 ? (v & 15u) : (v >> 4);
    };
    auto hi2 = [&](int i) -> unsigned {
      const int h = i >> 7, c = (i & 127) >> 5, l = i & 31;
      return (byte(128 + 32 * h + l) >> (2 * c)) & 3u;
    };
    for (int g = 0; g < 4; ++g) {
      const int ln = 16 * g + r;
      // scale byte j: k-steps with s >> 2 == j >> 1 and (s >> 1) & 1 == j & 1
      for (int j = 0; j < 4; ++j) {
        const int gg = (j >= 2 ? 2 : 0) + (g >> 1);
        rec[4 * ln + j] = (uint8_t)byte(192 + 4 * gg + 2 * (j & 1) + (g & 1));
      }
      // low nibbles where a Q4_K record keeps them: byte 8 (s & 1) + p of a
      // chunk, low nibble for step s, high nibble for step s + 2
      for (int j = 0; j < 16; ++j) {
        const int s = j >> 3, p = j & 7;
        rec[kTileQ0 + 16 * ln + j] = (uint8_t)(low4(lane_col(g, s, p)) | (low4(lane_col(g, s + 2, p)) << 4));
        rec[kTileQ1 + 16 * ln + j] = (uint8_t)(low4(lane_col(g, s + 4, p)) | (low4(lane_col(g, s + 6, p)) << 4));
      }
      unsigned hw[4] = {0u, 0u, 0u, 0u};
      for (int s = 0; s < 8; ++s)
        for (int q = 0; q < 4; ++q)
          for (int e = 0; e < 2; ++e)
            hw[s >> 1] |= hi2(lane_col(g, s, kPair[q][e])) << (8 * (s & 1) + 2 * q + 16 * e);
      for (int i = 0; i < 4; ++i) *(unsigned *)(rec + kTileQH + 16 * ln + 4 * i) = hw[i];
    }
    rec[kTileQ6D + 2 * r] = (uint8_t)byte(208);
    rec[kTileQ6D + 2 * r + 1] = (uint8_t)byte(209);
  }
}

// ---------------------------------------------------------------------------
// Target probability rows for the stochastic verify: p = softmax(z) per row,
// z = l / T after the optional soft cap l -> cap * tanh(l / cap). Two
// passes over chunks of kSmChunk logits (grid: chunks x rows):
//  1. each chunk's max of z and its sum of exp(z - chunk max) -> partials;
//  2. each chunk combines its row's partials (row max M,
//     S = sum_c s_c exp(m_c - M)) and writes p = exp(z - M) / S.
// Every reduction runs in a fixed order, so results are deterministic.
constexpr int kSmThreads = 256;
constexpr int kSmPer = 16;  // logits per thread
constexpr int64_t kSmChunk = (int64_t)kSmThreads * kSmPer;

__device__ __forceinline__ float sm_z(float l, float inv_cap, float cap, float temperature) {
  if (cap > 0.0f) l = cap * tanhf(l * inv_cap);
  return l / temperature;
}

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(kSmThreads) void kq_softmax_partial_kernel(const float *__restrict__ logits, int64_t n,
                                                                        float temperature, float cap,
                                                                        float2 *__restrict__ part) {
  __shared__ float red[4];
  const int64_t c = blockIdx.x, row = blockIdx.y, chunks = gridDim.x;
  const float *l = logits + row * n;
  const int64_t base = c * kSmChunk;
  const float inv_cap = cap > 0.0f ? 1.0f / cap : 0.0f;
  float z[kSmPer];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kSmPer; ++j) {
    const int64_t i = base + (int64_t)j * kSmThreads + threadIdx.x;
    z[j] = i < n ? sm_z(l[i], inv_cap, cap, temperature) : -INFINITY;
    mx = fmaxf(mx, z[j]);
  }
  mx = block_max(mx, red);
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kSmPer; ++j) sum += z[j] == -INFINITY ? 0.0f : expf(z[j] - mx);
  sum = block_sum(sum, red);
  if (threadIdx.x == 0) part[row * chunks + c] = float2{mx, sum};
}

__global__ __launch_bounds__(kSmThreads) void kq_softmax_write_kernel(const float *__restrict__ logits, int64_t n,
                                                                      float temperature, float cap,
                                                                      const float2 *__restrict__ part,
                                                                      float *__restrict__ probs) {
  const int64_t c = blockIdx.x, row = blockIdx.y, chunks = gridDim.x;
  const float2 *pr = part + row * chunks;
  // Row max and denominator: lane j takes partials j, j + 64, ... (loads in
  // parallel across the wave), then an xor butterfly across the wave. Max
  // and add are commutative, so every lane of every wave ends with the same
  // bits; the order is fixed, so results are the same on every run.
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  for (int64_t q = lane; q < chunks; q += 64) m = fmaxf(m, pr[q].x);
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float s = 0.0f;
  for (int64_t q = lane; q < chunks; q += 64) {
    const float2 v = pr[q];
    s += v.x == -INFINITY ? 0.0f : v.y * expf(v.x - m);
  }
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  const float *l = logits + row * n;
  float *p = probs + row * n;
  const int64_t base = c * kSmChunk;
  const float inv_cap = cap > 0.0f ? 1.0f / cap : 0.0f;
#pragma unroll
  for (int j = 0; j < kSmPer; ++j) {
    const int64_t i = base + (int64_t)j * kSmThreads + threadIdx.x;
    if (i < n) p[i] = expf(sm_z(l[i], inv_cap, cap, temperature) - m) / s;
  }
}

int softmax_chunks(int64_t n) { return (int)((n + kSmChunk - 1) / kSmChunk); }

int launch_softmax(const float *logits, int m, int64_t n, float temperature, float cap, float *part, float *probs,
                   void *stream) {
  const dim3 grid((unsigned)softmax_chunks(n), (unsigned)m);
  hipLaunchKernelGGL(kq_softmax_partial_kernel, grid, dim3(kSmThreads), 0, (hipStream_t)stream, logits, n,
                     temperature, cap, (float2 *)part);
  hipLaunchKernelGGL(kq_softmax_write_kernel, grid, dim3(kSmThreads), 0, (hipStream_t)stream, logits, n,
                     temperature, cap, (const float2 *)part, probs);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Read probe: every 16-byte chunk of a buffer is loaded once, workgroup b
// streaming its own contiguous slab (four 1 KB wave loads in flight per
// wave), XOR-folded, and one word per workgroup is written so the loads are
// not dead. Measures the HBM read rate the weight stream can reach.
__global__ __launch_bounds__(256) void kq_stream_probe_kernel(const u32x4 *__restrict__ p, int64_t chunks,
                                                              unsigned *__restrict__ sink) {
  const int64_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < chunks ? b0 + per : chunks;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 a0 = p[i], a1 = p[i + 256], a2 = p[i + 512], a3 = p[i + 768];
    acc ^= a0 ^ a1 ^ a2 ^ a3;
  }
  for (; i < b1; i += 256) acc ^= p[i];
  unsigned v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off, 64);
  __shared__ unsigned s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

int launch_stream_probe(const uint8_t *p, int64_t chunks, unsigned *sink, int blocks, void *stream) {
  hipLaunchKernelGGL(kq_stream_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)p, chunks, sink);
  return (int)hipGetLastError();
}

int launch_tile(const uint8_t *w, int64_t n, int64_t k, uint8_t *out, void *stream, int fmt) {
  const int64_t kb = k / kQK;
  const int64_t n_tiles = (n + 15) / 16;
  if (fmt == kFmtQ4) {
    const int64_t total = kb * n_tiles * 144;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(kq_tile_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w, n, kb,
                       n_tiles, out);
  } else {
    const int64_t blocks = (kb * n_tiles * 16 + 255) / 256;
    if (fmt == kFmtQ5)
      hipLaunchKernelGGL(kq_tile_kq_kernel<kFmtQ5>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w,
                         n, kb, n_tiles, out);
    else
      hipLaunchKernelGGL(kq_tile_kq_kernel<kFmtQ6>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w,
                         n, kb, n_tiles, out);
  }
  return (int)hipGetLastError();
}

int launch_stage(const float *x, int m, int64_t k, uint8_t *staged, unsigned *ctrl, int64_t n_groups,
                 void *stream) {
  const int64_t blocks = k / kQK;
  hipLaunchKernelGGL(kq_stage_kernel, dim3((unsigned)blocks, (unsigned)row_slices(m)), dim3(256), 0,
                     (hipStream_t)stream, x, m, k, staged, ctrl, n_groups);
  return (int)hipGetLastError();
}

int launch_fill(unsigned *p, int64_t n_words, void *stream, unsigned value) {
  int64_t blocks = (n_words + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(kq_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p,
                     n_words, value);
  return (int)hipGetLastError();
}

// The fixed workspace of kq_verify_argmax_accept_noalloc: one copy per GPU.
// Host code never uses the array's name as a device address; it uses the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[KQ_NOALLOC_MAX_BYTES];

int noalloc_workspace(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int read_device_word(const unsigned *dev, unsigned *host, void *stream) {
  hipError_t e = hipMemcpyAsync(host, dev, sizeof(unsigned), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  return (int)e;
}

// out[i] = rows[i][tokens[i]] (the accept tests' p_i[d_i]); a token outside
// [0, n) gives a NaN.
__global__ __launch_bounds__(256) void kq_gather_kernel(const float *__restrict__ rows, int64_t n,
                                                        const int32_t *__restrict__ tokens, int count,
                                                        float *__restrict__ out) {
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= count) return;
  const int32_t t = tokens[i];
  out[i] = (t >= 0 && (int64_t)t < n) ? rows[(int64_t)i * n + t] : __builtin_nanf("");
}

int launch_gather(const float *rows, int64_t n, const int32_t *tokens, int count, float *out, void *stream) {
  hipLaunchKernelGGL(kq_gather_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     rows, n, tokens, count, out);
  return (int)hipGetLastError();
}

int launch_gemv(const GemvLaunch &a, void *stream) {
  const dim3 grid((unsigned)a.g.n_wg);
  hipStream_t st = (hipStream_t)stream;
  if (a.chain || a.chain_single) {
    if (a.g.rows != kCwRows) return (int)hipErrorInvalidConfiguration;  // row groups of the chain geometry
    const dim3 block(64 * (kCwW + kCwP));
    if (a.chain_single) {
      // one phase, m <= 16, plain products of Q4_K weights
      if (a.verify || a.g.ms != 1 || a.x_rec != (unsigned)kStageBytes ||
          layout_fmt(a.layout) != kFmtQ4)
        return (int)hipErrorInvalidConfiguration;
      if (a.layout == KQ_LAYOUT_ROWS)
        hipLaunchKernelGGL((kq_chain_kernel<true, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((kq_chain_kernel<false, true>), grid, block, 0, st, a);
    } else if (a.layout == KQ_LAYOUT_ROWS) {
      hipLaunchKernelGGL((kq_chain_kernel<true, false>), grid, block, 0, st, a);
    } else {
      hipLaunchKernelGGL((kq_chain_kernel<false, false>), grid, block, 0, st, a);
    }
    return (int)hipGetLastError();
  }
  const int fmt = layout_fmt(a.layout);
  switch (a.g.ms * 1048576 + fmt * 65536 + a.g.waves * 4096 + a.g.tpw * 256 + a.g.bi * 16 + a.g.depth) {
#define KQ_CASE(F_, W_, T_, BI_, D_, MS_)                                                                    \
  case MS_ * 1048576 + F_ * 65536 + W_ * 4096 + T_ * 256 + BI_ * 16 + D_:                                    \
    if (F_ == kFmtQ4 && a.layout == KQ_LAYOUT_ROWS)                                                          \
      hipLaunchKernelGGL((kq_gemv_kernel<W_, T_, BI_, D_, F_, MS_, F_ == kFmtQ4>), grid, dim3(64 * W_), 0, st, \
                         a);                                                                                 \
    else                                                                                                     \
      hipLaunchKernelGGL((kq_gemv_kernel<W_, T_, BI_, D_, F_, MS_, false>), grid, dim3(64 * W_), 0, st, a);  \
    break;
    KQ_CASE(kFmtQ4, 8, 2, 4, 4, 1)
    KQ_CASE(kFmtQ4, 8, 1, 4, 4, 1)
    KQ_CASE(kFmtQ4, 8, 1, 2, 4, 1)
    KQ_CASE(kFmtQ4, 8, 2, 2, 4, 1)
    KQ_CASE(kFmtQ4, 4, 1, 1, 4, 1)
    KQ_CASE(kFmtQ4, 12, 1, 4, 4, 1)
    KQ_CASE(kFmtQ4, 4, 2, 2, 3, 1)
    KQ_CASE(kFmtQ4, 4, 2, 1, 3, 1)
    KQ_CASE(kFmtQ5, 8, 1, 4, 4, 1)
    KQ_CASE(kFmtQ5, 12, 1, 4, 4, 1)
    KQ_CASE(kFmtQ5, 8, 2, 4, 4, 1)
    KQ_CASE(kFmtQ6, 8, 1, 4, 4, 1)
    KQ_CASE(kFmtQ6, 12, 1, 4, 4, 1)
    KQ_CASE(kFmtQ6, 8, 2, 4, 4, 1)
    KQ_CASE(kFmtQ4, 8, 2, 2, 3, 2)
    KQ_CASE(kFmtQ5, 8, 2, 2, 3, 2)
    KQ_CASE(kFmtQ6, 8, 2, 2, 3, 2)
    KQ_CASE(kFmtQ4, 8, 2, 1, 2, 3)
    KQ_CASE(kFmtQ4, 8, 2, 1, 2, 4)
    KQ_CASE(kFmtQ5, 8, 2, 1, 2, 3)
    KQ_CASE(kFmtQ5, 8, 2, 1, 2, 4)
    KQ_CASE(kFmtQ6, 8, 2, 1, 2, 3)
    KQ_CASE(kFmtQ6, 8, 2, 1, 2, 4)
#undef KQ_CASE
    default: return (int)hipErrorInvalidConfiguration;
  }
  return (int)hipGetLastError();
}

// Workgroups of the chain kernel that the current device holds at once
// (resident blocks per CU times CUs), or a negative HIP error.
int chain_capacity() {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kq_chain_kernel<false, false>, 64 * (kCwW + kCwP), 0);
  if (e != hipSuccess) return -(int)e;
  return per_cu * cus;
}

}  // namespace kq
