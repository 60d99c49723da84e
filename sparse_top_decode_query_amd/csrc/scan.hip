// Plane-prefix scan (Fathom summary, bit-plane paragraph; per-token cost
// noted in its closing paragraph on HBM-resident scans).
//
// Score of token i under a plan (depth t_j, group query qbar):
//   s_i = sum_{t_j>0} qbar_j * (off_bj + scale_bj * (c_ij * 2^(4-t_j) + (2^(4-t_j)-1)/2))
// with c_ij the t_j-bit prefix code.  Since c * 2^(4-t) = sum_{p<t} bit_p * 2^(3-p),
// every plane bit carries a weight that does not depend on t:
//   s_i = C_b + sum_{t_j>p} bit_pij * 2^(3-p) * w_bj,   w_bj = qbar_j * scale_bj
//   C_b = sum_{t_j>0} qbar_j * off_bj + (qbar_j * (2^(4-t_j)-1)/2) * scale_bj
//
// Mapping onto CDNA: one lane owns one 32-token word of the planes, so every
// plane row is read as 64 consecutive dwords per wave (256-byte coalesced
// vector loads, each byte once), and the lane's 32 tokens share one 64-token
// block, so the weights w_bj are per-lane values.  Tokens i and i+16 of the
// word are handled together: one AND moves their t-bit codes into the low and
// high 16-bit halves of one register (cut from per-channel code registers,
// see use_chan), and a code pattern c read as an fp16 is the denormal
// c * 2^-24 -- exact -- so one v_fma_mix_f32 per token and channel adds
// c * (w_bj * 2^(24+4-t)) to a float32 accumulator: about 1.5 instructions
// per token and channel instead of one extract and one multiply-add per bit.
// The float32 constant C_b is accumulated alongside.
//
// Each channel's metadata and plane words come from a ring of buffers, three
// to six channels deep, to keep loads in flight.  Scores leave through LDS:
// lane l's 32 scores are consecutive tokens, so stores straight from the
// lanes would scatter 16-byte pieces 128 bytes apart; staged in LDS, every
// store instruction writes 1 KB of consecutive tokens (this alone cut the
// kernel's time by a sixth).
//
// Optionally the maximum score of every 64-token block is written as well
// (the two lanes of a block combine theirs), and the maximum of every group
// of kGroupBlocks blocks (16 lanes combine theirs); top-k selection uses them
// to skip blocks that cannot hold a winner.
//
// A growing cache: plane rows hold n_cap tokens, the first n are scored, and
// n need not be a multiple of 64.  Score rows are n rounded up to 64 long;
// the tokens past n in the open block score -inf, so they never reach a block
// maximum or the top-k.
#include "common.hpp"
#include "plan_dev.hpp"

namespace sdq {

constexpr int kScanWaves = 4;
constexpr int kTok = 32;                 // tokens per lane (one plane word)
constexpr int kGroupBlocks = SDQ_GROUP_BLOCKS;   // 64-token blocks per group maximum
static_assert(kGroupBlocks == 8, "a group is the 16 words of a quarter wave");

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int T>
struct ChanData {
  uint32_t mw;          // scale | offset << 16
  uint32_t W[T];        // this lane's word of planes 0..T-1
};

// Where a lane's loads come from: bounds-checked buffers over the head's
// planes and metadata, a fixed per-lane byte offset, and per-channel offsets
// that are wave-uniform (scalar registers), so addressing costs no vector
// instruction.
struct ScanSrc {
  __amdgpu_buffer_rsrc_t planes, meta;
  uint32_t plane_off, meta_off;   // this lane's word / block, in bytes
  uint32_t row_bytes, mrow_bytes;   // one plane row (n_cap/8 bytes), one metadata row (n_cap/16)
};

template <int T>
__device__ __forceinline__ void load_chan(ChanData<T>& d, const ScanSrc& src, int j) {
  d.mw = __builtin_amdgcn_raw_buffer_load_b32(src.meta, src.meta_off, uint32_t(j) * src.mrow_bytes, 0);
  const uint32_t base = uint32_t(j) * 4u * src.row_bytes;
#pragma unroll
  for (int p = 0; p < T; ++p)
    d.W[p] = __builtin_amdgcn_raw_buffer_load_b32(src.planes, src.plane_off, base + uint32_t(p) * src.row_bytes, 0);
}

// (a & m) | (b & ~m) as one v_bfi_b32, kept as written (left to itself the
// compiler rebuilds the selects below as masks and ORs, twice the work).
__device__ __forceinline__ uint32_t bfi32(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
  return r;
}

// Adds one channel's contribution to the 32 scores of the lane's word.
// q2 = qbar_j * 2^(28-t): with the fp16 scale it gives the weight of a t-bit
// code read as an fp16 denormal (c * 2^-24).
//
// Token pair (i, i+16) takes its two t-bit codes from one register: the
// codes sit at bit `pos` of the low and of the high half, pos = i for pairs
// 0..7 and i - 8 for pairs 8..15.  A half holding c << pos (< 2^11) reads as
// the fp16 value c * 2^(pos-24) exactly, so acc[i] collects 2^pos times its
// true sum; the factor is removed once at the end.  A pair costs one AND and
// two fma_mix.
//
// The registers the pairs are cut from: for t = 1 the plane word itself (and
// a copy shifted down by 8 for pairs 8..15).  For t >= 2 the codes of all
// tokens i of one residue class i mod S (S = 2 for t = 2, else 4; S >= t, so
// the codes of one class do not overlap) sit whole at bits [i, i+t) of one
// register z: bit x of z comes from plane t-1-s, s = (x - class) mod S, that
// plane pre-shifted so that token x-s lands on x.  Each class register costs
// t-1 bit selects, so a channel costs about 2S(t-1) + 2t + 16 bit
// instructions instead of 16t + 2t.
template <int T>
__device__ __forceinline__ void use_chan(const ChanData<T>& d, float qv, float qm, float q2,
                                         float& C, float (&acc)[kTok]) {
  const float sc = half_bits_to_f32(d.mw);
  const float off = half_bits_to_f32(d.mw >> 16);
  C = __builtin_fmaf(off, qv, C);
  C = __builtin_fmaf(sc, qm, C);
  const float w = sc * q2;
  auto pair = [&](int i, uint32_t src) {
    const int pos = i < 8 ? i : i - 8;
    uint32_t x = src & (((1u << T) - 1u) * 0x00010001u << pos);
    asm("" : "+v"(x));                 // keep x whole: its halves feed op_sel
    acc[i] = __builtin_fmaf(half_bits_to_f32(x), w, acc[i]);
    acc[i + 16] = __builtin_fmaf(half_bits_to_f32(x >> 16), w, acc[i + 16]);
  };
  if constexpr (T == 1) {
    const uint32_t lo = d.W[0], hi = d.W[0] >> 8;
#pragma unroll
    for (int i = 0; i < 16; ++i) pair(i, i < 8 ? lo : hi);
  } else {
    constexpr int S = T == 2 ? 2 : 4;
    constexpr uint32_t M0 = S == 2 ? 0x55555555u : 0x11111111u;   // positions of class 0
    uint32_t A[T], B[T];     // plane p: token x's bit at x + t-1-p (A) and x - 8 + t-1-p (B)
#pragma unroll
    for (int p = 0; p < T; ++p) {
      A[p] = d.W[p] << (T - 1 - p);
      B[p] = d.W[p] >> (8 - (T - 1 - p));
    }
    uint32_t za[S], zb[S];   // class registers for pairs 0..7 (za) and 8..15 (zb)
#pragma unroll
    for (int r = 0; r < S; ++r) {
      uint32_t va = A[0], vb = B[0];           // offset s = t-1 (and s >= t, never read)
#pragma unroll
      for (int s = T - 2; s >= 0; --s) {
        const uint32_t m = M0 << ((r + s) % S);
        va = bfi32(m, A[T - 1 - s], va);
        vb = bfi32(m, B[T - 1 - s], vb);
      }
      za[r] = va;
      zb[r] = vb;
      asm("" : "+v"(za[r]), "+v"(zb[r]));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) pair(i, i < 8 ? za[i % S] : zb[i % S]);
  }
}

// A ring of D channel buffers keeps D-1 channels' plane words and metadata in
// flight while one is accumulated (deeper or shallower rings measured
// slower).  The ring is indexed with compile-time slots, so its registers
// never move.
template <int T>
struct RingDepth {
  static constexpr int D = T == 1 ? 6 : (T == 2 ? 4 : 3);
};

// The channels of depth T at list slots a, a + S, a + 2S, ... below end (S = 1,
// or the number of waves sharing a tile, each taking every S-th channel).
// Full turns of the ring are straight-line code (D accumulations, each
// followed by the refill of its slot and a scheduling barrier), so the
// refills stay where they are written and each accumulation waits only for
// its own slot; refills past the end re-read the run's last channel (an L1
// hit).  The last partial turn only drains the ring.
template <int T, int S>
__device__ __forceinline__ void accum_run(int a, int end, const float4* s_ch,
                                          const ScanSrc& src, float& C, float (&acc)[kTok]) {
  constexpr int D = RingDepth<T>::D;
  if (a >= end) return;
  const int last = a + (end - 1 - a) / S * S;        // the last slot this wave takes
  auto fetch = [&](ChanData<T>& d, int x) {
    x = x < last ? x : last;
    load_chan<T>(d, src, __builtin_amdgcn_readfirstlane(__float_as_int(s_ch[x].w)));
  };
  ChanData<T> ring[D];
#pragma unroll
  for (int k = 0; k < D; ++k) fetch(ring[k], a + k * S);
  const int cnt = (last - a) / S + 1;
  const int turns = cnt / D;
  for (int it = 0; it < turns; ++it) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const int x = a + k * S;
      const float4 ch = s_ch[x];
      use_chan<T>(ring[k], ch.x, ch.y, ch.z, C, acc);
      fetch(ring[k], x + D * S);
      // Without this the scheduler hoists the bit work of every slot to the
      // top of the turn, which waits for all of the ring's loads and drains
      // it; with it a slot waits only for its own loads.
      __builtin_amdgcn_sched_barrier(0);
    }
    a += D * S;
  }
  const int rem = cnt - turns * D;
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const int x = a + k * S;
    if (k < rem) {
      const float4 ch = s_ch[x];
      use_chan<T>(ring[k], ch.x, ch.y, ch.z, C, acc);
    }
  }
}

// Plan inputs of the fused kernel (every workgroup derives its head's plan).
struct PlanIn {
  const float* q;
  const float* var;
  int Hgrp, budget;
  uint8_t* depth_out;     // optional copies of the plan, written by the first
  float* qbar_out;        // workgroup of each head
};

// MODE 0: plan read from depth/qbar; 1: water-filling plan; 2: uniform plan.
// SPLIT false: each wave scores its own 64 words (2048 tokens) over every
// active channel.  SPLIT true (short rows, too few words to fill the GPU
// with one wave each): the workgroup's waves share one 64-word tile, wave v
// takes every kScanWaves-th channel of each depth run, and the partial sums
// meet in LDS, so a tile's dependent chain of load turns is kScanWaves times
// shorter.
template <int MODE, bool SPLIT>
__global__ __launch_bounds__(kScanWaves * 64) void fathom_scan_kernel(
    const uint32_t* __restrict__ planes, const uint32_t* __restrict__ meta,
    const uint8_t* __restrict__ depth, const float* __restrict__ qbar, int n, int nb64, int n_cap,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ group_max,
    PlanIn pin) {
  // the active channels in depth order (4 first): qbar_j, its offset weight,
  // its code weight (see use_chan) and the channel index j, one 16-byte
  // read a channel
  __shared__ float4 s_ch[kHeadDim];
  __shared__ int s_run[5];          // list slots where depth 4, 3, 2, 1 start; s_run[4] = A
  // each wave's 2048 scores in token order (rows of 32 padded to 36 floats)
  __shared__ float4 s_out[kScanWaves][64 * 9];
  // Which head and tile this workgroup takes.  The dispatcher hands
  // consecutive workgroups to successive CUs, so with one head per grid row
  // each CU would hold the same tile of heads of one parity (0, 2, 4, 6 or
  // 1, 3, 5, 7 at 2^20 tokens), and one such set measured 6 us slower than
  // the other.  Instead, in every other pair of grid rows the two heads
  // swap, and each pair's tiles rotate by a quarter row, so a CU's
  // workgroups mix heads and token ranges (2^20 tokens: 0.2, 0.9 and 1.8 us
  // faster at B = 47, 56 and 92).  Short rows keep the plain order.
  int g = blockIdx.y, bx = blockIdx.x;
  if constexpr (!SPLIT) {
    const int r = g >> 1;
    if ((r & 1) && (g ^ 1) < int(gridDim.y)) g ^= 1;
    bx = int((unsigned(bx) + unsigned(r) * (gridDim.x >> 2)) % gridDim.x);
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  if (wave == 0) {
    // active channels sorted by depth (4 first); depths outside 1..4 are unread
    int t0, t1;
    float qv0, qv1;
    if constexpr (MODE == 0) {
      // depth and qbar in one round trip
      t0 = depth[size_t(g) * kHeadDim + lane];
      t1 = depth[size_t(g) * kHeadDim + lane + 64];
      qv0 = qbar[size_t(g) * kHeadDim + lane];
      qv1 = qbar[size_t(g) * kHeadDim + lane + 64];
    } else {
      // s_out is not used before the scores, so it lends the plan its scratch
      // (384 words)
      const HeadPlan p = plan_head<MODE == 2>(pin.q, pin.var, g, pin.Hgrp, pin.budget,
                                              reinterpret_cast<uint32_t*>(&s_out[0][0]));
      t0 = p.d0;
      t1 = p.d1;
      qv0 = p.a0;
      qv1 = p.a1;
      if (bx == 0 && pin.depth_out) {
        pin.depth_out[size_t(g) * kHeadDim + lane] = uint8_t(t0);
        pin.depth_out[size_t(g) * kHeadDim + lane + 64] = uint8_t(t1);
        pin.qbar_out[size_t(g) * kHeadDim + lane] = p.a0;
        pin.qbar_out[size_t(g) * kHeadDim + lane + 64] = p.a1;
      }
    }
    // Slots of the active channels, sorted by depth (4 first) and within a
    // depth by channel, from two packed wave scans: byte 4-L of x0 (x1)
    // counts channel lane (lane + 64) at depth L.
    const int x0 = (t0 >= 1 && t0 <= 4) ? 1 << (8 * (4 - t0)) : 0;
    const int x1 = (t1 >= 1 && t1 <= 4) ? 1 << (8 * (4 - t1)) : 0;
    const int i0 = wave_incl_scan(x0), i1 = wave_incl_scan(x1);
    const uint32_t n0 = uint32_t(wave_last(i0)), n1 = uint32_t(wave_last(i1));
    // byte f of pre: channels in runs 0..f (depth 4..4-f); at most 128, so
    // the byte-wise sums never carry
    const uint32_t pre = (n0 + n1) * 0x01010101u;
    auto place = [&](int t, int j, int before, float qv) {
      const int f = 4 - t;                       // run of depth t
      const int run0 = f == 0 ? 0 : int((pre >> (8 * (f - 1))) & 0xFFu);
      const int slot = run0 + (j >= 64 ? int((n0 >> (8 * f)) & 0xFFu) : 0) +
                       ((before >> (8 * f)) & 0xFF);
      s_ch[slot] = make_float4(qv, qv * (float((1 << (4 - t)) - 1) * 0.5f),
                               qv * float(1u << (28 - t)), __int_as_float(j));
    };
    if (x0) place(t0, lane, i0 - x0, qv0);
    if (x1) place(t1, lane + 64, i1 - x1, qv1);
    if (lane == 0) {
      s_run[0] = 0;
      s_run[1] = int(pre & 0xFFu);
      s_run[2] = int((pre >> 8) & 0xFFu);
      s_run[3] = int((pre >> 16) & 0xFFu);
      s_run[4] = int(pre >> 24);                 // A
    }
  }
  __syncthreads();
  const int A = __builtin_amdgcn_readfirstlane(s_run[4]);

  const size_t nw = size_t(nb64) * 2;                            // words scored (n rounded up to 64)
  const size_t nw_cap = size_t(n_cap) / 32;                       // words per plane row
  const int tile = SPLIT ? bx : bx * kScanWaves + wave;
  const int wd = tile * 64 + lane;                                // this lane's 32-token word
  if (tile * 64 >= int(nw)) return;                               // whole wave past the end
  const bool valid = wd < int(nw);
  const int wdc = valid ? wd : int(nw) - 1;                       // loads stay in bounds
  const int b = wdc >> 1;
  ScanSrc src;
  src.row_bytes = uint32_t(nw_cap) * 4u;
  src.mrow_bytes = uint32_t(n_cap / 64) * 4u;
  src.planes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(planes + size_t(g) * kHeadDim * 4 * nw_cap), (short)0,
      int(kHeadDim * 4 * src.row_bytes), 0x00020000);
  src.meta = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(meta + size_t(g) * kHeadDim * (n_cap / 64)), (short)0,
      int(kHeadDim * src.mrow_bytes), 0x00020000);
  src.plane_off = uint32_t(wdc) * 4u;
  src.meta_off = uint32_t(b) * 4u;

  // Channels are sorted by depth, so four fixed-depth runs cover them and the
  // accumulators never change registers.
  float C = 0.0f;
  float acc[kTok];
#pragma unroll
  for (int i = 0; i < kTok; ++i) acc[i] = 0.0f;
  const int r0 = __builtin_amdgcn_readfirstlane(s_run[0]), r1 = __builtin_amdgcn_readfirstlane(s_run[1]);
  const int r2 = __builtin_amdgcn_readfirstlane(s_run[2]), r3 = __builtin_amdgcn_readfirstlane(s_run[3]);
  constexpr int S = SPLIT ? kScanWaves : 1;
  const int v = SPLIT ? wave : 0;
  // A CU runs four workgroups at once and its arbiter favours the oldest
  // waves, so left alone the youngest workgroup does most of its work last,
  // nearly alone.  Each wave lowers its priority as its share of the work
  // (about t+2 units per channel of depth t) passes a quarter, a half and
  // three quarters, so lagging waves go first and the CU's waves end closer
  // together (measured 0.2-0.4 us faster at 2^20 tokens).
  const int work = (r1 - r0) * 6 + (r2 - r1) * 5 + (r3 - r2) * 4 + (A - r3) * 3 + 1;
  auto lower_priority = [&](int done) {
    const int q = done * 4 / work;
    if (q == 1) __builtin_amdgcn_s_setprio(2);
    else if (q == 2) __builtin_amdgcn_s_setprio(1);
    else if (q >= 3) __builtin_amdgcn_s_setprio(0);
  };
  __builtin_amdgcn_s_setprio(3);
  accum_run<4, S>(r0 + v, r1, s_ch, src, C, acc);
  lower_priority((r1 - r0) * 6);
  accum_run<3, S>(r1 + v, r2, s_ch, src, C, acc);
  lower_priority((r1 - r0) * 6 + (r2 - r1) * 5);
  accum_run<2, S>(r2 + v, r3, s_ch, src, C, acc);
  lower_priority((r1 - r0) * 6 + (r2 - r1) * 5 + (r3 - r2) * 4);
  accum_run<1, S>(r3 + v, A, s_ch, src, C, acc);
  if constexpr (SPLIT) {
    // waves 1.. hand their partial sums to wave 0, which adds them in wave
    // order (the staging rows of waves 1.. are free until then)
    if (wave > 0) {
      float* part = reinterpret_cast<float*>(s_out[wave]);
#pragma unroll
      for (int i = 0; i < kTok; ++i) part[i * 64 + lane] = acc[i];
      part[kTok * 64 + lane] = C;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < kScanWaves; ++w) {
      const float* part = reinterpret_cast<const float*>(s_out[w]);
#pragma unroll
      for (int i = 0; i < kTok; ++i) acc[i] += part[i * 64 + lane];
      C += part[kTok * 64 + lane];
    }
  }

  float sv[kTok];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kTok; ++i) {
    const int pos = (i & 15) < 8 ? (i & 15) : (i & 15) - 8;    // acc[i] holds 2^pos x its sum
    sv[i] = __builtin_fmaf(acc[i], __builtin_bit_cast(float, uint32_t(127 - pos) << 23), C);
  }
  const int wbase = tile * 64;                                    // first word of the tile
  if ((wbase + 64) * kTok > n) {                                  // the wave holds tokens past n
#pragma unroll
    for (int i = 0; i < kTok; ++i) sv[i] = wd * kTok + i < n ? sv[i] : -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < kTok; ++i) m = fmaxf(m, sv[i]);
  // Scores leave through LDS so that every store instruction writes 1 KB of
  // consecutive tokens (lane l holds tokens 32l..32l+31 of the wave's range).
  float4* so = s_out[wave];
#pragma unroll
  for (int v = 0; v < kTok / 4; ++v)
    so[lane * 9 + v] = make_float4(sv[4 * v], sv[4 * v + 1], sv[4 * v + 2], sv[4 * v + 3]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int nvalid = int(nw) - wbase < 64 ? int(nw) - wbase : 64; // words of the wave in range
  float4* dst = reinterpret_cast<float4*>(scores + size_t(g) * nb64 * 64 + size_t(wbase) * kTok);
#pragma unroll
  for (int v = 0; v < kTok / 4; ++v) {
    const int f = v * 64 + lane;                                  // float4 index in the wave's range
    const int word = f >> 3;                                      // 8 float4 per word
    // non-temporal: the scores are read once, by another kernel, so they
    // need not stay in this XCD's L2 (measured 0.2-1 us off the launch)
    if (word < nvalid)
      __builtin_nontemporal_store(__builtin_bit_cast(f32x4, so[word * 9 + (f & 7)]),
                                  reinterpret_cast<f32x4*>(&dst[f]));
  }
  if (block_max || group_max) {
    m = fmaxf(m, __shfl_xor(m, 1, 64));                          // the block's two words
    if (block_max && valid && (lane & 1) == 0) block_max[size_t(g) * nb64 + b] = m;
    if (group_max) {
      // 16 words from a multiple of 16: lanes past the end hold -inf
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      m = fmaxf(m, __shfl_xor(m, 4, 64));
      m = fmaxf(m, __shfl_xor(m, 8, 64));
      const int ngr = (nb64 + kGroupBlocks - 1) / kGroupBlocks;
      if (valid && (lane & 15) == 0) group_max[size_t(g) * ngr + (wd >> 4)] = m;
    }
  }
}

}  // namespace sdq

using namespace sdq;

// Rows too short to give every CU its share of one-wave tiles: the waves of
// a workgroup share a tile instead (at most 1024 tiles over all KV heads,
// i.e. 4096 waves, 16 per CU).
static bool scan_split(int G, int nb64) {
  const long long tiles = (long long)G * ((2LL * nb64 + 63) / 64);
  return tiles <= 1024;
}

static int scan_checks(const char* nm, const uint32_t* planes, const uint32_t* meta, int G,
                       int d, int n, int n_cap, const float* scores) {
  SDQ_REQUIRE(planes && meta && scores, "%s: null pointer", nm);
  SDQ_REQUIRE(G >= 1, "%s: G=%d must be >= 1", nm, G);
  SDQ_REQUIRE(n_cap >= 64 && n_cap % 64 == 0, "%s: n_cap=%d must be a positive multiple of 64", nm,
              n_cap);
  SDQ_REQUIRE(n >= 1 && n <= n_cap, "%s: n=%d must be in [1, n_cap=%d]", nm, n, n_cap);
  SDQ_REQUIRE(n_cap < (1 << 25), "%s: n_cap=%d must be below 2^25 (a head's planes fit 2 GiB)", nm,
              n_cap);
  SDQ_REQUIRE(d == kHeadDim, "%s: d=%d unsupported (only 128)", nm, d);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(scores) % 16 == 0, "%s: scores must be 16-byte aligned", nm);
  return SDQ_OK;
}

extern "C" int fathom_scan(const uint32_t* planes, const uint32_t* meta, const uint8_t* depth,
                           const float* qbar, int G, int d, int n, int n_cap, float* scores,
                           float* block_max, float* group_max, hipStream_t stream) {
  SDQ_REQUIRE(depth && qbar, "fathom_scan: null pointer");
  if (const int rc = scan_checks("fathom_scan", planes, meta, G, d, n, n_cap, scores)) return rc;
  const int nb64 = (n + 63) / 64;
  if (scan_split(G, nb64))
    hipLaunchKernelGGL((fathom_scan_kernel<0, true>), dim3(cdiv(size_t(nb64) * 2, 64), G),
                       dim3(kScanWaves * 64), 0, stream, planes, meta, depth, qbar, n, nb64, n_cap,
                       scores, block_max, group_max, PlanIn{});
  else
    hipLaunchKernelGGL((fathom_scan_kernel<0, false>), dim3(cdiv(size_t(nb64) * 2, kScanWaves * 64), G),
                       dim3(kScanWaves * 64), 0, stream, planes, meta, depth, qbar, n, nb64, n_cap,
                       scores, block_max, group_max, PlanIn{});
  return check_launch("fathom_scan");
}

extern "C" int fathom_plan_scan(const float* q, const float* key_var, int H_grp, int budget,
                                int uniform, const uint32_t* planes, const uint32_t* meta, int G,
                                int d, int n, int n_cap, uint8_t* depth, float* qbar, float* scores,
                                float* block_max, float* group_max, hipStream_t stream) {
  SDQ_REQUIRE(q && key_var, "fathom_plan_scan: null pointer");
  SDQ_REQUIRE((depth == nullptr) == (qbar == nullptr),
              "fathom_plan_scan: depth and qbar must both be given or both be null");
  SDQ_REQUIRE(H_grp >= 1, "fathom_plan_scan: H_grp=%d must be >= 1", H_grp);
  SDQ_REQUIRE(budget >= 0, "fathom_plan_scan: budget/channel count %d must be >= 0", budget);
  SDQ_REQUIRE(!uniform || budget <= d, "fathom_plan_scan: n_channels=%d exceeds d=%d", budget, d);
  if (const int rc = scan_checks("fathom_plan_scan", planes, meta, G, d, n, n_cap, scores)) return rc;
  const int nb64 = (n + 63) / 64;
  const PlanIn pin{q, key_var, H_grp, budget, depth, qbar};
  const bool split = scan_split(G, nb64);
  const dim3 grid(cdiv(size_t(nb64) * 2, split ? 64 : kScanWaves * 64), G);
  const dim3 block(kScanWaves * 64);
  if (uniform && split)
    hipLaunchKernelGGL((fathom_scan_kernel<2, true>), grid, block, 0, stream, planes, meta, nullptr,
                       nullptr, n, nb64, n_cap, scores, block_max, group_max, pin);
  else if (uniform)
    hipLaunchKernelGGL((fathom_scan_kernel<2, false>), grid, block, 0, stream, planes, meta, nullptr,
                       nullptr, n, nb64, n_cap, scores, block_max, group_max, pin);
  else if (split)
    hipLaunchKernelGGL((fathom_scan_kernel<1, true>), grid, block, 0, stream, planes, meta, nullptr,
                       nullptr, n, nb64, n_cap, scores, block_max, group_max, pin);
  else
    hipLaunchKernelGGL((fathom_scan_kernel<1, false>), grid, block, 0, stream, planes, meta, nullptr,
                       nullptr, n, nb64, n_cap, scores, block_max, group_max, pin);
  return check_launch("fathom_plan_scan");
}
