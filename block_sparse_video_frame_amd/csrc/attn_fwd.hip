// attn_fwd: forward pass of frame-aligned block-sparse attention on gfx950.
//
// The method (vatt-ghern.pages.dev "deep-heygen-avatar-iv-trillium-tpu",
// sections 把 block 縮到 16 and 拿掉 softmax 的序列相依; bytechap "How it
// works"; cloudcurated Wall 2 and Wall 3):
//   * the key set of a query tile is a list of intervals whose ends are
//     multiples of 16 tokens on frame edges, so every key block is either
//     fully attended or absent: no mask predicate, no padding, no extra scan;
//   * softmax either keeps the standard running max (rescaling the running
//     sum and accumulator whenever the max grows), or fixes each row's shift
//     before the key loop to the Cauchy-Schwarz bound scale*|q_i|*max|k_j|
//     from precomputed norms, so the loop never rescales; heads whose bound
//     is too loose take the running-max path (here a second instantiation of
//     the same kernel template, launched right after the first).
//
// gfx950 design (not the TPU kernel's):
//   * A workgroup computes one query tile of up to 256 rows of one (batch,
//     head) at a time: 8 waves x 32 query rows.  A wave keeps its Q rows in
//     VGPRs for the whole tile (the bound path keeps Q pre-multiplied by
//     scale*log2(e)).
//   * S^T = K * Q^T and O^T = V^T * P^T with v_mfma_f32_32x32x16_bf16 (fp32
//     accumulate).  With that orientation lane (n, h) of a 32x32 accumulator
//     owns query n, so the row shift, the row sum and the rescale factor of a
//     query live in the lanes that own it: P feeds the second MFMA straight
//     from registers and the bound path needs no cross-lane traffic at all.
//   * Keys stream through LDS in stages of 64 (K and V, [64][D] bf16 each),
//     four buffers deep with loads issued two stages ahead.  Stages are filled
//     by LDS-direct buffer loads (global -> LDS, no VGPR round trip); a stage
//     may gather rows from several intervals, and the last stage of a tile
//     holds a multiple of 16 keys.  16-byte chunks are XOR-swizzled by row so
//     both the K reads and the transposing V reads (ds_read_b64_tr_b16) are
//     free of bank conflicts.
//   * The upper four waves run half a stage behind the lower four (PV of the
//     previous stage before QK of this one) so the two halves' MFMA and
//     exp/VALU phases interleave on each SIMD.
//   * A tile of at most 64 rows (the short last tile of a frame) runs thin:
//     four waves, one per SIMD, hold the same 32 rows; each takes one 32-key
//     half of every other stage, and the four merge their partial sums
//     through LDS at the end.  Such a tile otherwise has one busy wave.
//   * The bound path runs persistent: one workgroup per CU takes tiles from
//     its accelerator die's queue of the launch order, then from the other
//     dies' queues, since the dies do not run at equal speed.
//   * exp is v_exp_f32 on base-2 scores; the tail stage zeroes the scores of
//     missing 16-key groups (a per-group select, never a per-element mask).
#include "bsvf_device.h"
#include "bsvf_internal.h"

#include <cfloat>
#include <mutex>
#include <type_traits>

namespace bsvf {
namespace {

constexpr int BK = 64;  // keys per LDS stage
#ifndef ONLINE_NQB
#define ONLINE_NQB 1
#define ONLINE_NW 8
#endif
#ifndef BOUND_NQB
#define BOUND_NQB 1
#define BOUND_NW 8
#endif
// s_waitcnt immediate that waits for every outstanding vector memory access
// (vmcnt 0) and leaves the export and LDS counters alone.
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The fixed shift is the bound times this margin, which keeps it above every
// score the kernel computes: the fp32 dot products and the fp32 norms each
// carry rounding error below D * 2^-24 relative for D <= 128, far inside 2^-8.
constexpr float kBoundMargin = 1.0f + 1.0f / 256.0f;
// Smallest row sum a checked tile keeps (2^ATTN_CHECK_LOG2_L).
constexpr float kCheckMinL = 0x1p-100f;
static_assert(ATTN_CHECK_LOG2_L == -100.0f, "kCheckMinL is 2^ATTN_CHECK_LOG2_L");
// A checked tile's shift lies ATTN_CHECK_SHIFT_NATS below the bound (log2 units).
constexpr float kCheckShift2 = ATTN_CHECK_SHIFT_NATS * kLog2e;
// Bound rows come in two kinds.  Where the slack bound is at most
// ATTN_PRESCALE_NATS, the bound loop keeps Q multiplied by scale*log2(e) and
// rounded to bf16 once, and starts the score accumulator at -m, so the MFMA
// yields the exponent directly (no FMA per score).  That rounding moves a
// score by up to 2^-9 of |q||k| (scale*|q||k| is at most half the slack
// bound), which near the eligibility limit would cost most of the error
// budget.  Rows with a looser bound keep Q exact and take the exponent with
// one FMA per score: they run on the online loop with its running max
// switched off (a fixed shift).
// s_getreg operand for the XCC id hardware register (id 20, bits 31:0)
constexpr int kHwRegXccId = (31 << 11) | 20;

// Read-only inputs (block lists, norms) are read through constant-address-
// space pointers: the compiler then treats every load from them as invariant
// and keeps uniform ones on the scalar unit, whichever way the pointer came.
typedef __attribute__((address_space(4))) const int32_t ci32;
typedef __attribute__((address_space(4))) const float cf32;

struct FwdArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  float* shift_out;
  int64_t sq[3], sk[3], sv[3], so[3];
  int32_t B, H, N;
  float scale;
  float c2;  // scale * log2(e)
  const int32_t* q_tiles;
  const int32_t* kv_ptr;
  const int32_t* kv_iv;
  int32_t n_qt, nnz, block_q;
  const int32_t* work_order;
  int32_t n_work;
  int32_t n_xcd;            // queues in work_order (persistent launch)
  int32_t* work_ctr;        // their slot counters, then a done count (persistent launch)
  const float* q_norm;
  const float* k_gmax;
  const float* head_max;
  int32_t mode;
  int32_t gate;             // persistent online-only launch: kGateNone or kGateOnline
  int32_t* head_path_out;
  // frame mask of the frame-unaware layout (kernels built with MASK only)
  const int32_t* kv_flag;   // per interval: 1 = some (row, key) pair masked
  int32_t frame_T;          // tokens per frame
  int32_t win_lo, win_hi;   // key frame - query frame allowed in [win_lo, win_hi]
  uint32_t gbits[2];        // global key frames, bit f of the 64-bit word
};


__device__ __forceinline__ bf16x8 to_bf16x8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    f32x2 f = {p[i], p[i + 1]};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    r[i] = b[0];
    r[i + 1] = b[1];
  }
  return r;
}

// p0 + p1 + acc for a packed bf16 pair (one v_dot2 with (1, 1)): the row sum
// adds exactly the rounded probabilities the P*V product uses.  A v_dot2
// cannot issue while a matrix instruction is running; plain fp32 adds can.
__device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

// Workgroup-wide OR of one flag per wave, through the first NW words of the
// stage array; every wave calls it.  The first barrier puts every wave past
// its last use of the stage array (no stage copy is in flight by then), the
// last keeps later copies off the words until every wave has read them.
template <int NW>
__device__ __forceinline__ bool group_any(bool flag, u16* smem, int wave, int lane) {
  int* word = reinterpret_cast<int*>(smem);
  __syncthreads();
  if (lane == 0) word[wave] = flag ? 1 : 0;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) any |= word[w];
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(any) != 0;
}

__device__ __forceinline__ bool interval_ok(int ks, int kl, int N) {
  return ks >= 0 && kl > 0 && ((ks | kl) & 15) == 0 && ks <= N - kl;
}

// Stages in flight ahead of the one being consumed, and LDS buffers: the
// prefetch window, the stage being consumed, and the lagging half's previous
// stage (see run_tile).
constexpr int kPrefetch = 2;
constexpr int kBuffers = kPrefetch + 2;

template <int D, int NQB, int NW>
struct Cfg {
  static constexpr int NT = 64 * NW;
  static constexpr int BQ = 32 * NQB * NW;
  static constexpr int DC = D / 8;               // 16-byte chunks per K/V row
  static constexpr int KSTEPS = D / 16;          // MFMA k-steps of Q*K^T
  static constexpr int DBLK = D / 32;            // 32-wide output blocks
  static constexpr int REGION = BK * D;          // elements of K (or V) per stage
  static constexpr int STAGE = 2 * REGION;       // K + V elements per stage
  // Stage buffer x's K region starts BSTRIDE * x elements into the stage
  // array and its V region VOFF elements past its K.  At D = 128 a buffer is
  // K then V; at D = 64 the four K regions come first, then the four V
  // regions, so every buffer's offset within the K (or V) regions fits a
  // read's immediate offset (see Tile::kImm).
  static constexpr int BSTRIDE = D == 64 ? REGION : STAGE;
  static constexpr int VOFF = D == 64 ? kBuffers * REGION : REGION;
  static constexpr int LPW = DC / NW;            // 1 KiB direct loads per wave per region
  static_assert(LPW >= 1 && LPW * NW == DC, "tile shape");
};

// LDS layout of a stage: K rows then V rows, [64 keys][D] bf16 each, with the
// 16-byte chunk c of row r stored at chunk position c ^ swz(r).  LDS has 64
// four-byte banks; a 16-byte read is served 16 lanes at a time and an 8-byte
// (transposing) read 32 lanes at a time.  The swizzle spreads both the K
// operand reads (16 consecutive rows, one chunk) and the transposing V reads
// (4 consecutive rows x 4 adjacent chunks per 32 lanes) over all 64 banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int lds_off(int row, int col) {
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// Operand addresses as XOR forms.  A stage buffer starts at a multiple of its
// size (a power of two at least 16 times a row), so within it:
//   K operand of key block kb, k-step st (row 32kb + n, chunk 2st + hh):
//       ((buffer | kl) ^ 32st) + 32 * row_bytes * kb
//   transposing V read of key rows 32kb + 16kst + [0, 16), output block db:
//       (buffer | (vl[hi] ^ 64db)) + V region + row_bytes * (32kb + 16kst)
// with per-lane kl and vl[hi] from lane_offsets().  The swizzle XORs bits of
// the chunk index that the k-step (or output block) index only XORs into, so
// one XOR per operand replaces the row/column arithmetic and the rest folds
// into the read's immediate offset.
template <int D>
struct LaneOffsets {
  uint32_t kl;
  uint32_t vl[2];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane) {
  constexpr uint32_t RS = 2 * D;  // bytes per row
  const int n = lane & 31, hh = lane >> 5, t16 = lane & 15, g2 = (lane >> 4) & 1;
  LaneOffsets<D> o;
  const int s = swz<D>(n);
  o.kl = RS * n + 32 * (s >> 1) + 16 * (hh ^ (s & 1));
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int r16 = (4 * hh + (t16 >> 2) + 8 * hi) & 15;
    const int sv = swz<D>(r16);
    const int cl = 2 * g2 + ((t16 & 3) >> 1);
    o.vl[hi] = RS * r16 + 64 * (sv >> 2) + 16 * (cl ^ (sv & 3)) + 8 * (t16 & 1);
  }
  return o;
}

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ const lds_char* lds_bytes(const u16* smem) {
  return (const lds_char*)(smem);
}

// Buffer descriptor over one head's rows of K or V (raw buffer, byte
// offsets).  Reads at offsets past `bytes` return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const u16* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets of the LDS-DMA loads of a stage that is one
// contiguous run of 64 keys: key row `row` of the run at the chunk the swizzle
// puts at this lane's LDS slot.  The run's start enters as a scalar offset.
template <int D, int NQB, int NW>
struct DmaLanes {
  uint32_t k[Cfg<D, NQB, NW>::LPW];
  uint32_t v[Cfg<D, NQB, NW>::LPW];
  __device__ __forceinline__ void init(uint32_t ksn, uint32_t vsn, int wave, int lane) {
    using C = Cfg<D, NQB, NW>;
#pragma unroll
    for (int it = 0; it < C::LPW; ++it) {
      const int slot = (it * NW + wave) * 64 + lane;
      const int row = slot / C::DC, phys = slot % C::DC;
      const uint32_t col = (phys ^ swz<D>(row)) << 3;
      k[it] = 2u * (row * ksn + col);
      v[it] = 2u * (row * vsn + col);
    }
  }
};

// Direct global -> LDS copy of one stage that is a contiguous run of keys
// start .. start+63.  Each wave-wide load fills 1 KiB of LDS in lane order, so
// every lane fetches the chunk the swizzle places at its LDS slot.
template <int D, int NQB, int NW>
__device__ __forceinline__ void issue_stage_run(u16* ks, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                            const DmaLanes<D, NQB, NW>& dl, uint32_t ksn, uint32_t vsn,
                                            int start, int wave) {
  using C = Cfg<D, NQB, NW>;
  const uint32_t sk = 2u * (uint32_t)start * ksn, sv = 2u * (uint32_t)start * vsn;
#pragma unroll
  for (int it = 0; it < C::LPW; ++it) {
    const int blk = it * NW + wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(ks + blk * 512), 16, (int)dl.k[it], (int)sk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(ks + C::VOFF + blk * 512), 16, (int)dl.v[it],
                                             (int)sv, 0, 0);
  }
}

// A stage in general: the next 64 positions of the tile's keys, taken in
// order across its intervals (at most four, as every interval holds a
// multiple of 16 keys).  Position r < end[j] (first such j) is key base[j] + r;
// positions at or past `n` do not exist (only the tile's last stage is short).
struct StageDesc {
  int base[4];
  int end[4];
  int n;
};

// Direct global -> LDS copy of a general stage.  Positions past the stage's
// count re-load its last key (in bounds, finite); their probabilities are
// zeroed before use.
template <int D, int NQB, int NW>
__device__ __forceinline__ void issue_stage(u16* ks, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                            uint32_t ksn, uint32_t vsn, const StageDesc& sd, int wave,
                                            int lane) {
  using C = Cfg<D, NQB, NW>;
#pragma unroll
  for (int it = 0; it < C::LPW; ++it) {
    const int blk = it * NW + wave;
    const int slot = blk * 64 + lane;
    const int row = slot / C::DC, phys = slot % C::DC;
    const uint32_t col = (phys ^ swz<D>(row)) << 3;
    const int r = min(row, sd.n - 1);
    const int base = r < sd.end[0] ? sd.base[0] : r < sd.end[1] ? sd.base[1] : r < sd.end[2] ? sd.base[2] : sd.base[3];
    const uint32_t key = base + r;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(ks + blk * 512), 16, 2 * (key * ksn + col), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(ks + C::VOFF + blk * 512), 16,
                                             2 * (key * vsn + col), 0, 0, 0);
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// Transposing LDS read: within each 16-lane group, output lane i element j is
// element i % 4 of the 8 bytes addressed by lane 4j + i / 4.
__device__ __forceinline__ i16x4 ds_read_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// P*V: the transposing V reads (two per MFMA) start PV_AHEAD MFMAs before the
// MFMA that consumes them, so LDS latency hides behind matrix work.
#ifndef PV_AHEAD
#define PV_AHEAD 2
#endif
// K operand reads start KAHEAD MFMAs before their use in the fused step.
#ifndef KAHEAD
#define KAHEAD 3
#endif
template <int NMFMA>
__device__ __forceinline__ void pin_pv() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_AHEAD, 1);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
}

template <int D, int NQB, int NW, bool BOUNDQ>
struct Tile {
  using C = Cfg<D, NQB, NW>;
  using Scores = f32x16[2][NQB];
  using Probs = bf16x8[NQB][2][2];
  bf16x8 qreg[NQB][C::KSTEPS];
  f32x16 oacc[NQB][C::DBLK];
  float m2[NQB];    // row shift in log2 units (bound: fixed; online: running max)
  bool fixed;       // online loop with a fixed shift (the bound with exact Q): no max, no rescale
  float lsum[NQB];   // this lane half's share of the row sum
  float lsum2[NQB];  // a second running sum (the second pair of a chunk at D = 64,
                     // the odd probabilities at D = 128)
  // Row sums.  At D = 128 a stage has twice the matrix work per probability,
  // enough to hide two fp32 adds per pair under the MFMAs, and the sums add
  // the fp32 probabilities.  At D = 64 the vector unit is the tighter one and
  // a v_dot2 per pair sums them as rounded to bf16 for the P*V product.
  static constexpr bool kSumF32 = D == 128;
  int n, hh, lane;
  int fq[NQB];  // frame of this lane's query row (frame-unaware layout only)
  LaneOffsets<D> lof;
  static constexpr uint32_t RS = 2 * D;
  // At D = 64 the operand addresses within a buffer live in registers: the K
  // operand of k-step st at kx[st] = kl ^ 32st, the transposing V reads of
  // output block db at vx[hi][db] (from the start of the V regions).  A
  // buffer's byte offset `boff` (a multiple of the region size, above these
  // bits) then adds as the read's immediate offset wherever the walk knows
  // the buffer at compile time (see run_tile), so such a read needs no
  // address arithmetic.  At D = 128 each read forms its address with one XOR:
  // the twelve registers would spill in the combined kernel, and the XORs hide
  // under the stage's matrix work there.
  static constexpr bool kImm = D == 64;
  uint32_t kx[kImm ? C::KSTEPS : 1];
  uint32_t vx[2][kImm ? C::DBLK : 1];
  __device__ __forceinline__ void set_addresses() {
    if constexpr (kImm) {
#pragma unroll
      for (int st = 0; st < C::KSTEPS; ++st) kx[st] = lof.kl ^ (32u * st);
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) vx[hi][db] = 2u * C::VOFF + (lof.vl[hi] ^ (64u * db));
    }
  }
  // Called at the top of each step: the per-lane offsets count as new values
  // there, so the compiler does not hoist offset-plus-buffer sums for every
  // buffer out of the walk (which would hold one register per sum).
  __device__ __forceinline__ void renew_addresses() {
    if constexpr (kImm) {
#pragma unroll
      for (int st = 0; st < C::KSTEPS; ++st) asm volatile("" : "+v"(kx[st]));
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) asm volatile("" : "+v"(vx[hi][db]));
    }
  }

  // Byte address (less v_rows()) of the transposing V reads of output block
  // db, lane half `hi`, in the stage buffer at byte `boff`.
  __device__ __forceinline__ uint32_t v_address(uint32_t boff, int hi, int db) const {
    if constexpr (kImm) return boff + vx[hi][db];
    else return boff | (lof.vl[hi] ^ (64u * db));
  }
  __device__ __forceinline__ static constexpr uint32_t v_rows() { return kImm ? 0u : 2u * C::VOFF; }

  // K operand of block kb, k-step st, of the stage buffer at byte `boff`.
  __device__ __forceinline__ bf16x8 k_operand(const lds_char* sm, uint32_t boff, int kb, int st) const {
    if constexpr (kImm) return *(const volatile lds_bf16x8*)(sm + kx[st] + (boff + 32u * RS * kb));
    else return *(const volatile lds_bf16x8*)(sm + (((boff | lof.kl) ^ (32u * st)) + 32u * RS * kb));
  }

  // Score accumulators start at acc0[qb]: the bound loop starts at -m (its Q
  // already carries scale*log2(e)), so the MFMA yields the exponent directly;
  // the online loop (also running fixed shifts) at 0.
  __device__ __forceinline__ float acc0(int qb) const { return BOUNDQ ? -m2[qb] : 0.0f; }

  // S^T = K * Q^T for the 64 keys of a stage: lane (n, hh) gets keys
  // 32kb + 8i + 4hh + j (register 4i + j) of query n.
  __device__ __forceinline__ void scores(const lds_char* sm, uint32_t boff, Scores& s) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = acc0(qb);
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = k_operand(sm, boff, kb, st);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[qb][st], s[kb][qb], 0, 0, 0);
      }
  }

  // Probabilities of one stage as bf16 MFMA operands.  Bound: exp(s - m) with
  // the fixed shift, no max and no rescale.  Online: raise the running max;
  // alpha[qb] is the factor the accumulator still has to be rescaled by.
  // TAIL: only the first `nvalid` keys of the stage are real (a multiple of
  // 16, so keys 32kb + 8i .. +7 are all real or all missing).
  template <bool BOUND, bool TAIL>
  __device__ __forceinline__ void softmax(const Scores& s, Probs& pk, float (&alpha)[NQB], int nvalid,
                                          float c2) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      alpha[qb] = 1.0f;
      if (!BOUND && !fixed) {
        // Missing keys hold copies of a real key of this row, so they cannot
        // raise the max above a real score.
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m2[qb], mx * c2);
        // a row none of whose keys so far is attended (frame-unaware layout)
        // keeps m = -inf; shift by 0 then, so that nothing becomes NaN
        const float msafe = mnew == -INFINITY ? 0.0f : mnew;
        alpha[qb] = __builtin_amdgcn_exp2f(m2[qb] - msafe);
        m2[qb] = mnew;
        lsum[qb] *= alpha[qb];
        lsum2[qb] *= alpha[qb];
      }
      const float nm = m2[qb] == -INFINITY ? 0.0f : -m2[qb];
      float p[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          p[kb][r] = __builtin_amdgcn_exp2f(BOUND ? s[kb][qb][r] : fmaf(s[kb][qb][r], c2, nm));
      if constexpr (TAIL) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool live = 32 * kb + 8 * i < nvalid;
#pragma unroll
            for (int j = 0; j < 4; ++j) p[kb][4 * i + j] = live ? p[kb][4 * i + j] : 0.0f;
          }
      }
      float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pk[qb][kb][0] = to_bf16x8(p[kb]);
        pk[qb][kb][1] = to_bf16x8(p[kb] + 8);
        if constexpr (kSumF32) {
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            t0 += p[kb][r];
            t1 += p[kb][r + 1];
          }
        } else {
#pragma unroll
          for (int kst = 0; kst < 2; ++kst) {
            const u32x4 w = __builtin_bit_cast(u32x4, pk[qb][kb][kst]);
            t0 = add_pair(w[0], t0); t1 = add_pair(w[1], t1);
            t0 = add_pair(w[2], t0); t1 = add_pair(w[3], t1);
          }
        }
      }
      lsum[qb] += t0 + t1;
    }
  }

  // The softmax of a full stage (`cur`) fused with the Q*K^T MFMAs of the
  // next stage (`nxt`, K operands from `ks`).  The two are independent, so the
  // code is laid out as one chunk per MFMA -- a K operand read three MFMAs
  // ahead, the MFMA, then a slice of the softmax -- and sched_barrier keeps
  // the compiler from regrouping the chunks: the matrix core runs while the
  // vector ALU works.  Results equal softmax<BOUND, false> then scores().
  template <bool BOUND>
  __device__ __forceinline__ void softmax_and_scores(const Scores& cur, const lds_char* sm, uint32_t boff, Scores& nxt,
                                                     Probs& pk, float (&alpha)[NQB], float c2) {
    constexpr int NM = 2 * C::KSTEPS;       // MFMAs per 32 queries (st, kb)
    constexpr int EPM = 32 / NM;            // softmax elements per MFMA (2 or 4)
    constexpr int AHEAD = KAHEAD;
    float nm[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      alpha[qb] = 1.0f;
      if (!BOUND && !fixed) {
        float mx = cur[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m2[qb], mx * c2);
        // a row none of whose keys so far is attended (frame-unaware layout)
        // keeps m = -inf; shift by 0 then, so that nothing becomes NaN
        const float msafe = mnew == -INFINITY ? 0.0f : mnew;
        alpha[qb] = __builtin_amdgcn_exp2f(m2[qb] - msafe);
        m2[qb] = mnew;
        lsum[qb] *= alpha[qb];
        if constexpr (EPM > 2 || kSumF32) lsum2[qb] *= alpha[qb];
      }
      nm[qb] = m2[qb] == -INFINITY ? 0.0f : -m2[qb];
    }
    // MFMA i accumulates block kbn(i) of the next stage: the first half of the
    // chunks fills block 1 while block 0 of `cur` is being consumed, the second
    // half fills block 0 once those registers are free (48 live score
    // registers per 32 queries instead of 64).
    auto kbn = [](int i) { return i < C::KSTEPS ? 1 : 0; };
    auto stn = [](int i) { return i % C::KSTEPS; };
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) nxt[1][qb][r] = acc0(qb);
    // K operand reads are volatile so they issue AHEAD MFMAs before their use
    // instead of being sunk next to it.
    bf16x8 kf[NM];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i)
      kf[i] = k_operand(sm, boff, kbn(i), stn(i));
    uint32_t pw[NQB][2][8];  // packed bf16 pairs: [qb][kb][r / 2]
    // The softmax of chunk i is skewed over three chunks -- its exps in chunk
    // i, their conversion to bf16 in chunk i+1, the row-sum update in chunk
    // i+2 -- so no instruction waits on a result issued just before it; the
    // wave's matrix and vector work then interleave without stalls.  Pairs
    // go straight into the running row sums (the second one where a chunk
    // holds two pairs), with no per-stage partial sums to start and fold.
    // The fp32 sums of D = 128 are added in chunk i+1, beside the conversion
    // (kept to chunk i+2, the probabilities would need more registers).
    float pe[NM][NQB][EPM];        // chunk i's probabilities (fp32)
    uint32_t pp[NM][NQB][EPM / 2];  // chunk i's packed bf16 pairs
    // The exponent of each score, s * scale * log2(e) - m, is taken one chunk
    // ahead of its exp (xe), so the exp never waits on the FMA before it.
    constexpr bool kFma = !BOUND;
    float xe[NM][NQB][EPM];
    auto arg = [&](int i) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int e = 0; e < EPM; ++e) {
          const int el = i * EPM + e, kb = el >> 4, r = el & 15;
          xe[i][qb][e] = kFma ? fmaf(cur[kb][qb][r], c2, nm[qb]) : cur[kb][qb][r];
        }
    };
    if constexpr (kFma) arg(0);
#pragma unroll
    for (int i = 0; i < NM + 2; ++i) {
      if (i < NM) {
        if (i + AHEAD < NM) {
          const int j = i + AHEAD;
          kf[j] = k_operand(sm, boff, kbn(j), stn(j));
        }
        if (i == C::KSTEPS) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) nxt[0][qb][r] = acc0(qb);
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          nxt[kbn(i)][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qreg[qb][stn(i)], nxt[kbn(i)][qb], 0, 0, 0);
        if constexpr (!kFma) arg(i);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int e = 0; e < EPM; ++e) {
            pe[i][qb][e] = __builtin_amdgcn_exp2f(xe[i][qb][e]);
            // keep this slice here: without a use at this point the
            // compiler sinks the whole softmax below the MFMAs
            asm volatile("" : "+v"(pe[i][qb][e]));
          }
        if constexpr (kFma) {
          if (i + 1 < NM) {
            arg(i + 1);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
              for (int e = 0; e < EPM; ++e) asm volatile("" : "+v"(xe[i + 1][qb][e]));
          }
        }
      }
      if (i >= 1 && i <= NM) {
        const int c = i - 1;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int e = 0; e < EPM; e += 2) {
            const int el = c * EPM + e, kb = el >> 4, r = el & 15;
            f32x2 f = {pe[c][qb][e], pe[c][qb][e + 1]};
            uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
            asm volatile("" : "+v"(w));
            pp[c][qb][e >> 1] = w;
            pw[qb][kb][r >> 1] = w;
            if constexpr (kSumF32) {
              lsum[qb] += pe[c][qb][e];
              lsum2[qb] += pe[c][qb][e + 1];
            }
          }
      }
      if (i >= 2) {
        const int c = i - 2;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
          for (int e = 0; e < EPM; e += 2) {
            if constexpr (kSumF32) {
              // summed in chunk i+1
            } else if ((e >> 1) & 1) {
              lsum2[qb] = add_pair(pp[c][qb][e >> 1], lsum2[qb]);
            } else {
              lsum[qb] = add_pair(pp[c][qb][e >> 1], lsum[qb]);
            }
          }
          asm volatile("" : "+v"(lsum[qb]), "+v"(lsum2[qb]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kst = 0; kst < 2; ++kst) {
          u32x4 w = {pw[qb][kb][4 * kst], pw[qb][kb][4 * kst + 1], pw[qb][kb][4 * kst + 2], pw[qb][kb][4 * kst + 3]};
          pk[qb][kb][kst] = __builtin_bit_cast(bf16x8, w);
        }
    }
  }

  // Frame mask of one stage of the frame-unaware layout: keys k0 .. k0+63 (a
  // contiguous run; at most one frame edge in it as tokens_per_frame >= 64).
  // Scores of keys this lane's row may not attend, and of positions at or
  // past `nvalid`, become -inf.  Key position p = 32kb + 8i + 4hh + j holds
  // register 4i + j of block kb.
  __device__ __forceinline__ void apply_mask(Scores& s, const FwdArgs& a, int k0, int nvalid) const {
    const int T = a.frame_T;
    const int f0 = k0 / T;
    const int edge = (f0 + 1) * T - k0;  // first position in frame f0 + 1
    const uint64_t gb = (uint64_t)a.gbits[0] | ((uint64_t)a.gbits[1] << 32);
    const bool g0 = f0 < 64 && ((gb >> f0) & 1), g1 = f0 + 1 < 64 && ((gb >> (f0 + 1)) & 1);
    const int thr = edge - 4 * hh, lim = nvalid - 4 * hh;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int d = f0 - fq[qb];
      const bool ok0 = (d >= a.win_lo && d <= a.win_hi) || g0;
      const bool ok1 = (d + 1 >= a.win_lo && d + 1 <= a.win_hi) || g1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pb = 32 * kb + 8 * (r >> 2) + (r & 3);
          const bool keep = (pb >= thr ? ok1 : ok0) && pb < lim;
          s[kb][qb][r] = keep ? s[kb][qb][r] : -INFINITY;
        }
    }
  }

  // Online path: apply the pending rescale to the accumulator, skipped when
  // no row of the wave raised its max.
  __device__ __forceinline__ void rescale(const float (&alpha)[NQB]) {
    if (fixed) return;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
      if (__any(alpha[qb] != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) oacc[qb][db] *= alpha[qb];
      }
  }

  // O^T += V^T * P^T: k-step (kb, kst) covers keys 32kb + 16kst + [0, 16);
  // lane (n, hh) needs V[32kb + 16kst + 8(e/4) + 4hh + e%4][32db + n] as its
  // element e, which two transposing reads deliver: source lane t of each
  // 16-lane group addresses key row (... + 4hh + t/4) at columns
  // 32db + 16((lane/16)%2) + 4(t%4) .. +3.
  __device__ __forceinline__ void pv(const lds_char* sm, uint32_t boff, const Probs& pk) {
    uint32_t va[2][C::DBLK];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) va[h2][db] = v_address(boff, h2, db);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kst = 0; kst < 2; ++kst)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
          const uint32_t rows = v_rows() + RS * (32 * kb + 16 * kst);
          const i16x4 lo4 = ds_read_tr16(sm + va[0][db] + rows);
          const i16x4 hi4 = ds_read_tr16(sm + va[1][db] + rows);
          const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pk[qb][kb][kst], oacc[qb][db], 0, 0, 0);
        }
  }

  // ---- Thin tiles (at most 64 rows; see run_thin): a wave takes one 32-key
  // block `kb` of a stage.  Register j of a half holds key
  // 32kb + 8(j/4) + 4hh + j%4, as in the full-stage layout.
  using Half = f32x16;
  using HalfProbs = bf16x8[2];

  __device__ __forceinline__ void scores_half(const lds_char* sm, uint32_t boff, int kb, Half& s) const {
    static_assert(NQB == 1, "thin tiles take one row group per wave");
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = acc0(0);
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(sm, boff, kb, st), qreg[0][st], s, 0, 0, 0);
  }

  // Online path: raise the running max by this half's scores; returns the
  // factor the accumulator has to be rescaled by.
  __device__ __forceinline__ float raise_max(const Half& s, float c2) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m2[0], mx * c2);
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m2[0] - msafe);
    m2[0] = mnew;
    lsum[0] *= alpha;
    return alpha;
  }

  // Probabilities of one half stage (see softmax).  TAIL: only the first
  // `nvalid` keys of the whole stage are real.
  template <bool BOUND, bool TAIL>
  __device__ __forceinline__ void softmax_half(const Half& s, HalfProbs& pk, float& alpha, int nvalid, float c2,
                                               int kb) {
    alpha = (BOUND || fixed) ? 1.0f : raise_max(s, c2);
    const float nm = m2[0] == -INFINITY ? 0.0f : -m2[0];
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(BOUND ? s[r] : fmaf(s[r], c2, nm));
    if constexpr (TAIL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = 32 * kb + 8 * i < nvalid;
#pragma unroll
        for (int j = 0; j < 4; ++j) p[4 * i + j] = live ? p[4 * i + j] : 0.0f;
      }
    }
    pk[0] = to_bf16x8(p);
    pk[1] = to_bf16x8(p + 8);
    float t0 = 0.0f, t1 = 0.0f;
    if constexpr (kSumF32) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        t0 += p[r];
        t1 += p[r + 1];
      }
    } else {
#pragma unroll
      for (int kst = 0; kst < 2; ++kst) {
        const u32x4 w = __builtin_bit_cast(u32x4, pk[kst]);
        t0 = add_pair(w[0], t0); t1 = add_pair(w[1], t1);
        t0 = add_pair(w[2], t0); t1 = add_pair(w[3], t1);
      }
    }
    lsum[0] += t0 + t1;
  }

  __device__ __forceinline__ void rescale_half(float alpha) {
    if (!fixed && __any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) oacc[0][db] *= alpha;
    }
  }

  // O^T += V^T * P^T over key block kb of a stage.
  __device__ __forceinline__ void pv_half(const lds_char* sm, uint32_t boff, int kb, const HalfProbs& pk) {
    uint32_t va[2][C::DBLK];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) va[h2][db] = v_address(boff, h2, db);
    const uint32_t base = v_rows() + RS * 32 * kb;
#pragma unroll
    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        const uint32_t rows = base + RS * 16 * kst;
        const i16x4 lo4 = ds_read_tr16(sm + va[0][db] + rows);
        const i16x4 hi4 = ds_read_tr16(sm + va[1][db] + rows);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pk[kst], oacc[0][db], 0, 0, 0);
      }
  }
};

// s_waitcnt immediate that waits until at most n vector memory accesses of
// this wave are outstanding (they complete in order), leaving the export and
// LDS counters alone.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

#ifndef ISSUE_LAG
#define ISSUE_LAG 1
#endif

// Cuts the tile's valid intervals into consecutive 64-key stages (scalar,
// uniform state).  Intervals outside [0, N) or not 16-aligned are skipped.
// Start and length of interval e.  e is the same in every lane; saying so
// lets the compiler read the list with scalar loads (a vector load's wait
// would also wait for every stage copy in flight).
__device__ __forceinline__ void interval_at(const ci32* kv_iv, int e, int& ks, int& kl) {
  const int u = __builtin_amdgcn_readfirstlane(e);
  ks = kv_iv[2 * u];
  kl = kv_iv[2 * u + 1];
}

struct KeyWalker {
  const ci32* kv_iv;
  int e, e1, N, cs, cl, off;
  bool more;

  __device__ __forceinline__ void seek() {
    for (; e < e1; ++e) {
      interval_at(kv_iv, e, cs, cl);
      if (interval_ok(cs, cl, N)) break;
    }
    more = e < e1;
    off = 0;
  }
  // Next stage.  Returns true when it is one contiguous run of 64 keys (the
  // common case), given by `start`; otherwise fills `d`.
  __device__ __forceinline__ bool next(StageDesc& d, int& start) {
    if (more && cl - off >= BK) {
      start = cs + off;
      off += BK;
      if (off >= cl) { ++e; seek(); }
      return true;
    }
    int pos = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (more && pos < BK) {
        const int take = min(cl - off, BK - pos);
        d.base[k] = cs + off - pos;
        pos += take;
        off += take;
        if (off >= cl) { ++e; seek(); }
      } else {
        d.base[k] = k ? d.base[k - 1] : 0;
      }
      d.end[k] = pos;
    }
    d.n = pos;
    return false;
  }
};

// The start key and mask flag of the stages in the order they are consumed
// (the frame-unaware layout, whose stages each lie inside one interval).
struct StageCursor {
  const ci32* kv_iv;
  const ci32* kv_flag;
  int e, e1, N, cs, cl, off;
  bool flag;

  __device__ __forceinline__ void seek() {
    for (; e < e1; ++e) {
      interval_at(kv_iv, e, cs, cl);
      if (interval_ok(cs, cl, N)) break;
    }
    if (e < e1) { off = 0; flag = kv_flag[__builtin_amdgcn_readfirstlane(e)] != 0; }
  }
  __device__ __forceinline__ void next(int& k0, bool& masked) {
    k0 = cs + off;
    masked = flag;
    off += BK;
    if (off >= cl) { ++e; seek(); }
  }
};

// Software-pipelined walk over the tile's stages with kBuffers LDS buffers
// (stage x lives in buffer x mod kBuffers).  Per iteration s, after one
// barrier, stage s+kPrefetch starts streaming in, and each wave runs F(s) --
// the softmax of stage s fused with the Q*K^T MFMAs of stage s+1 (VALU-heavy)
// -- and a P*V step (MFMA only).  The two waves that share a SIMD run them in
// opposite orders: the leading half of the workgroup does F(s) then P(s); the
// lagging half does P(s-1) then F(s).  One wave's vector work then overlaps
// the other's matrix work instead of both contending for the same unit.
// Every stage but the tile's last is full.
template <int D, int NQB, int NW, bool BOUND, bool LAG, bool MASK>
__device__ __forceinline__ void run_tile(const FwdArgs& a, const ci32* kv_iv, u16* smem,
                                         Tile<D, NQB, NW, BOUND>& T, const u16* kh, const u16* vh,
                                         int e0, int e1, int wave, bool active) {
  using C = Cfg<D, NQB, NW>;
  using TT = Tile<D, NQB, NW, BOUND>;
  // Stage copies are issued by the issuing waves only: the lagging half
  // (ISSUE_LAG), each wave taking twice the share, right after it has issued
  // the transposing V reads of its P*V step.  The compiler orders every LDS
  // read of that kind after all LDS-DMA copies the wave has in flight (it
  // cannot tell the buffers apart), so a wave that issued the copies before
  // its V reads would wait for them to land -- the full copy latency, every
  // stage.  Issued after the reads, the copies are waited for only at the
  // next stage's barrier, and the leading waves never wait on them.
  constexpr int IW = ISSUE_LAG ? NW / 2 : NW;  // issuing waves
  constexpr bool kIssuer = !ISSUE_LAG || LAG;
  using CI = Cfg<D, NQB, IW>;
  constexpr int LOADS = 2 * CI::LPW;  // vector memory ops per issuing wave per stage
  const int iwave = ISSUE_LAG ? wave - NW / 2 : wave;
  static_assert((kBuffers & (kBuffers - 1)) == 0, "buffer count must be a power of two");
  const uint32_t ksn = (uint32_t)a.sk[2], vsn = (uint32_t)a.sv[2];
  const __amdgpu_buffer_rsrc_t kr = head_rsrc(kh, 2u * (ksn * (uint32_t)(a.N - 1) + D));
  const __amdgpu_buffer_rsrc_t vr = head_rsrc(vh, 2u * (vsn * (uint32_t)(a.N - 1) + D));
  int total = 0;
  for (int e = e0; e < e1; ++e)
    if (interval_ok(kv_iv[2 * e], kv_iv[2 * e + 1], a.N)) total += kv_iv[2 * e + 1];
  if (total == 0) return;
  const int ns = (total + BK - 1) / BK, nlast = total - BK * (ns - 1);
  // stage x's K region (its V region lies VOFF elements on)
  auto kbuf = [&](int x) { return smem + (x & (kBuffers - 1)) * C::BSTRIDE; };
  // byte offset of stage x's K region within the stage array
  auto boff = [&](int x) { return (uint32_t)((x & (kBuffers - 1)) * C::BSTRIDE * 2); };
  const lds_char* sm = lds_bytes(smem);
  KeyWalker kw{kv_iv, e0, e1, a.N, 0, 0, 0, false};
  kw.seek();
  StageCursor cur_stage{kv_iv, (const ci32*)a.kv_flag, e0, e1, a.N, 0, 0, 0, false};
  if constexpr (MASK) cur_stage.seek();
  // frame mask of stage x (consumed in order), before its softmax
  auto mask_stage = [&](typename Tile<D, NQB, NW, BOUND>::Scores& sc_x, int x) {
    if constexpr (MASK) {
      int k0;
      bool masked;
      cur_stage.next(k0, masked);
      if (masked) T.apply_mask(sc_x, a, k0, x == ns - 1 ? nlast : BK);
    }
  };
  DmaLanes<D, NQB, IW> dl;
  if constexpr (kIssuer) dl.init(ksn, vsn, iwave, T.lane);
  auto issue = [&](int x) {
    StageDesc sd;
    int start;
    if (kw.next(sd, start)) issue_stage_run<D, NQB, IW>(kbuf(x), kr, vr, dl, ksn, vsn, start, iwave);
    else issue_stage<D, NQB, IW>(kbuf(x), kr, vr, ksn, vsn, sd, iwave, T.lane);
  };
  if constexpr (kIssuer) {
#pragma unroll
    for (int x = 0; x < kPrefetch; ++x)
      if (x < ns) issue(x);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm((kPrefetch - 1) * LOADS));  // stage 0 landed, if it was not alone
  if (ns < kPrefetch) __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  typename TT::Scores sc;
  if (active) T.scores(sm, boff(0), sc);
  typename TT::Probs pk;
  float alpha[NQB];
  // A step's buffers: stage st + rel is in buffer (st + rel) mod kBuffers.
  // The walk below runs the steps in groups of kBuffers with st a multiple of
  // kBuffers at the first (Phase J is st mod kBuffers, or -1 where unknown),
  // so the buffer offsets are compile-time constants that the operand reads
  // take as immediate offsets.
  auto step = [&](auto phase, int st, typename TT::Scores& cur, typename TT::Scores& nxt) {
    constexpr int J = decltype(phase)::value;
    T.renew_addresses();
    auto bo = [&](int rel) -> uint32_t {
      if constexpr (J >= 0) return (uint32_t)(((J + rel) & (kBuffers - 1)) * C::BSTRIDE * 2);
      else return boff(st + rel);
    };
    // Stage st+1 has landed (every wave): at most the stages after it are
    // still in flight.  Every wave is also done with the buffer stage
    // st+kPrefetch is about to overwrite.
    if (st + kPrefetch - 1 < ns) __builtin_amdgcn_s_waitcnt(wait_vm((kPrefetch - 2) * LOADS));
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    const bool more = st + kPrefetch < ns;
    if constexpr (!ISSUE_LAG) {
      if (more) issue(st + kPrefetch);
    }
    if (!active) {
      if constexpr (ISSUE_LAG && LAG) {
        if (more) issue(st + kPrefetch);
      }
      return;
    }
    mask_stage(cur, st);
    if constexpr (LAG) {
      if (st > 0) {
        T.pv(sm, bo(-1), pk);
        pin_pv<4 * C::DBLK * NQB>();
      }
      if constexpr (ISSUE_LAG) {
        __builtin_amdgcn_sched_barrier(0);
        if (more) issue(st + kPrefetch);
        __builtin_amdgcn_sched_barrier(0);
      }
      T.template softmax_and_scores<BOUND>(cur, sm, bo(1), nxt, pk, alpha, a.c2);
      if constexpr (!BOUND) T.rescale(alpha);
    } else {
      T.template softmax_and_scores<BOUND>(cur, sm, bo(1), nxt, pk, alpha, a.c2);
      if constexpr (!BOUND) T.rescale(alpha);
      T.pv(sm, bo(0), pk);
      pin_pv<4 * C::DBLK * NQB>();
    }
  };
  typename TT::Scores sn;
  static_assert(kBuffers == 4, "the walk runs its steps in groups of four");
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using PX = std::integral_constant<int, -1>;
  int st = 0;
  if constexpr (TT::kImm) {
    for (; st + 4 < ns; st += 4) {
      step(P0{}, st, sc, sn);
      step(P1{}, st + 1, sn, sc);
      step(P2{}, st + 2, sc, sn);
      step(P3{}, st + 3, sn, sc);
    }
  }
  for (; st + 2 < ns; st += 2) {
    step(PX{}, st, sc, sn);
    step(PX{}, st + 1, sn, sc);
  }
  if (st + 1 < ns) {
    step(PX{}, st, sc, sn);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) sc[kb][qb] = sn[kb][qb];
  }
  // Last stage (its copy was waited for at the top of the last iteration, or
  // before the loop when the tile has a single stage).
  if (!active) return;
  mask_stage(sc, ns - 1);
  if (LAG && ns > 1) T.pv(sm, boff(ns - 2), pk);
  if (nlast == BK) T.template softmax<BOUND, false>(sc, pk, alpha, BK, a.c2);
  else T.template softmax<BOUND, true>(sc, pk, alpha, nlast, a.c2);
  if constexpr (!BOUND) T.rescale(alpha);
  T.pv(sm, boff(ns - 1), pk);
}

// The walk of a thin tile (at most 64 rows).  It consumes two stages per
// step: wave w works on row group w/4, stage 2j + (w/2)%2 of step j, and key
// block kb = w%2 of that stage, so a 16-row tile keeps all four SIMDs busy.
// Waves past the tile's row groups only copy.  A step waits for its two
// stages, then refills the two buffers the previous step consumed.  At the
// end the four waves of a row group hold partial sums over disjoint keys: the
// three with (stage parity, kb) != (0, 0) hand theirs (accumulator, row sum,
// shift) to the fourth through the stage buffers, and it merges them in a
// fixed order (same shift on the bound path; rescaled to the largest running
// max on the online path).
template <int D, int NQB, int NW, bool BOUND>
__device__ __forceinline__ void run_thin(const FwdArgs& a, const ci32* kv_iv, u16* smem,
                                         Tile<D, NQB, NW, BOUND>& T, const u16* kh, const u16* vh, int e0, int e1,
                                         int wave, bool active) {
  using C = Cfg<D, NQB, NW>;
  using TT = Tile<D, NQB, NW, BOUND>;
  constexpr int LOADS = 2 * C::LPW;
  static_assert(kBuffers == 4 && NW == 8, "thin walk: two stages consumed, two in flight; 8 waves");
  const int kb = wave & 1, sp = (wave >> 1) & 1, part = wave & 3;
  const uint32_t ksn = (uint32_t)a.sk[2], vsn = (uint32_t)a.sv[2];
  const __amdgpu_buffer_rsrc_t kr = head_rsrc(kh, 2u * (ksn * (uint32_t)(a.N - 1) + D));
  const __amdgpu_buffer_rsrc_t vr = head_rsrc(vh, 2u * (vsn * (uint32_t)(a.N - 1) + D));
  int total = 0;
  for (int e = e0; e < e1; ++e)
    if (interval_ok(kv_iv[2 * e], kv_iv[2 * e + 1], a.N)) total += kv_iv[2 * e + 1];
  if (total == 0) return;
  const int ns = (total + BK - 1) / BK, nlast = total - BK * (ns - 1);
  auto kbuf = [&](int x) { return smem + (x & (kBuffers - 1)) * C::BSTRIDE; };
  auto boff = [&](int x) { return (uint32_t)((x & (kBuffers - 1)) * C::BSTRIDE * 2); };
  const lds_char* sm = lds_bytes(smem);
  KeyWalker kw{kv_iv, e0, e1, a.N, 0, 0, 0, false};
  kw.seek();
  DmaLanes<D, NQB, NW> dl;
  dl.init(ksn, vsn, wave, T.lane);
  auto issue = [&](int x) {
    StageDesc sd;
    int start;
    if (kw.next(sd, start)) issue_stage_run<D, NQB, NW>(kbuf(x), kr, vr, dl, ksn, vsn, start, wave);
    else issue_stage<D, NQB, NW>(kbuf(x), kr, vr, ksn, vsn, sd, wave, T.lane);
  };
#pragma unroll
  for (int x = 0; x < kBuffers; ++x)
    if (x < ns) issue(x);
  typename TT::Half sc;
  typename TT::HalfProbs pk;
  float alpha;
  for (int s0 = 0; s0 < ns; s0 += 2) {
    // Stages s0 and s0+1 landed (every wave).  Issued so far: stages 0-3 and
    // then two per step, i.e. up to min(max(3, s0+1), ns-1); the first step
    // leaves stages 2 and 3 in flight, later ones none.
    if (s0 == 0 && ns >= 4) __builtin_amdgcn_s_waitcnt(wait_vm(2 * LOADS));
    else if (s0 == 0 && ns == 3) __builtin_amdgcn_s_waitcnt(wait_vm(LOADS));
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // the previous step's two buffers are free again
    if (s0 > 0) {
      if (s0 + 2 < ns) issue(s0 + 2);
      if (s0 + 3 < ns) issue(s0 + 3);
    }
    const int st = s0 + sp;
    if (active && st < ns) {
      T.scores_half(sm, boff(st), kb, sc);
      if (st == ns - 1 && nlast != BK) T.template softmax_half<BOUND, true>(sc, pk, alpha, nlast, a.c2, kb);
      else T.template softmax_half<BOUND, false>(sc, pk, alpha, BK, a.c2, kb);
      if constexpr (!BOUND) T.rescale_half(alpha);
      T.pv_half(sm, boff(st), kb, pk);
      pin_pv<2 * C::DBLK>();
    }
  }
  // Every copy has landed (the last step waited for all of them) and, past
  // this barrier, no wave reads a stage buffer: the partials go anywhere in
  // the stage array.  Partial p of row group g: parts 1-3 of the group.
  __syncthreads();
  constexpr int NO = C::DBLK * 16;        // accumulator registers per lane
  constexpr int PSTRIDE = (NO + 2) * 64;  // floats per partial
  static_assert(2 * 3 * PSTRIDE * 4 <= kBuffers * C::STAGE * 2, "partials must fit in the stage buffers");
  float* const mb0 = reinterpret_cast<float*>(smem) + (wave >> 2) * 3 * PSTRIDE;
  if (active && part != 0) {
    float* mb = mb0 + (part - 1) * PSTRIDE;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) mb[(db * 16 + r) * 64 + T.lane] = T.oacc[0][db][r];
    mb[NO * 64 + T.lane] = T.lsum[0];
    mb[(NO + 1) * 64 + T.lane] = T.m2[0];
  }
  __syncthreads();
  if (active && part == 0) {
    float f[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (!BOUND) {
      float mp[4] = {T.m2[0], 0.0f, 0.0f, 0.0f};
      float m = mp[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        mp[q] = mb0[(q - 1) * PSTRIDE + (NO + 1) * 64 + T.lane];
        m = fmaxf(m, mp[q]);
      }
      const float msafe = m == -INFINITY ? 0.0f : m;
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = __builtin_amdgcn_exp2f(mp[q] - msafe);
      T.m2[0] = m;
    }
    float l = T.lsum[0] * f[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) l += mb0[(q - 1) * PSTRIDE + NO * 64 + T.lane] * f[q];
    T.lsum[0] = l;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float o = T.oacc[0][db][r] * f[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) o += mb0[(q - 1) * PSTRIDE + (db * 16 + r) * 64 + T.lane] * f[q];
        T.oacc[0][db][r] = o;
      }
  }
}

// What run_item did with an item.
enum ItemResult { kDeclined = 0, kDone = 1, kRetry = 2 };

// The per-head test's slack bound of head bh in nats: the largest score any
// of its rows can reach, 2 * scale * max|q| * max|k| (twice the largest
// possible distance between the shift and a score).
__device__ __forceinline__ float head_slack(float scale, const cf32* head_max, int bh) {
  return 2.0f * scale * head_max[2 * bh] * head_max[2 * bh + 1];
}

// In the per-head mode the persistent launch is two kernels on the same
// work: the online-only kernel, which has a register allocation of its own,
// then the combined kernel (both loops).  The first (kGateOnline) runs the
// items only when no head takes the bound loop, else the second does.
enum { kGateNone = 0, kGateOnline = 1 };

// One work item w (a query tile of one (batch, head)) on the softmax path
// BOUND, in the stage array `smem`.  Returns kDeclined, having written
// nothing, when the item takes the other path; kRetry, having written
// nothing, when it is a checked tile (mode 5) whose check failed -- the
// caller runs it again with `force_online`; kDone when it is done (or is no
// valid item).  All waves of the workgroup call it and return together,
// except that waves with no rows may return before the epilogue.  Only
// kernels built with CHECK (launched for mode 5) hold the check.
template <int D, int NQB, int NW, bool BOUND, bool MASK, bool CHECK, bool NODECLINE = false>
__device__ __forceinline__ int run_item(const FwdArgs& a, const ci32* q_tiles, const ci32* kv_ptr,
                                        const ci32* kv_iv, const cf32* k_gmax, const cf32* head_max,
                                        u16* smem, int w, bool force_online = false) {
  const cf32* q_norm = (const cf32*)a.q_norm;
  using C = Cfg<D, NQB, NW>;
  // The thread index is made opaque, so that the per-lane setup derived from
  // it is computed per item instead of being hoisted out of a persistent
  // workgroup's item loop and held in registers across it.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;

  const int total = a.n_qt * a.H * a.B;
  if (w < 0 || w >= total) return kDone;
  const int tile = w % a.n_qt, bh = w / a.n_qt;
  const int b = bh / a.H, h = bh % a.H;
  const int qs = q_tiles[2 * tile], nr = q_tiles[2 * tile + 1];
  if (qs < 0 || nr <= 0 || nr > C::BQ || nr > a.block_q || qs > a.N - nr) return kDone;
  int e0 = kv_ptr[tile], e1 = kv_ptr[tile + 1];
  e0 = max(0, min(e0, a.nnz));
  e1 = max(e0, min(e1, a.nnz));

  // Softmax path: uniform per workgroup; per head (modes 1, 2, 4) or per
  // tile (modes 3 and 5, which need the tile's largest query and key norms
  // first).  A slack bound within ATTN_PRESCALE_NATS takes the bound loop
  // (prescaled Q; not in mode 4, which never rounds Q); up to
  // ATTN_ELIGIBLE_NATS the online loop with the bound as a fixed shift
  // (exact Q); in mode 5, up to ATTN_CHECK_NATS the same, checked after the
  // fact (kCheck); beyond it the running max.  Forced mode: bound loop.  A
  // checked tile that failed runs again on the running max.
  enum { kOnline = 0, kExact = 1, kPre = 2, kCheck = 3 };
  // (Only kernels built with CHECK run mode 5.)
  const bool checked = CHECK && a.mode == ATTN_SOFTMAX_BOUND_CHECKED && !force_online;
  auto classify = [checked](float slack) {
    return slack <= ATTN_PRESCALE_NATS ? kPre
           : slack <= ATTN_ELIGIBLE_NATS ? kExact
           : checked && slack <= ATTN_CHECK_NATS ? kCheck
                                                 : kOnline;
  };
  const bool per_tile = a.mode == ATTN_SOFTMAX_BOUND_TILE || a.mode == ATTN_SOFTMAX_BOUND_CHECKED;
  int path = kOnline;
  if (a.mode == ATTN_SOFTMAX_BOUND_FORCED) {
    path = kPre;
  } else if (a.mode == ATTN_SOFTMAX_BOUND || a.mode == ATTN_SOFTMAX_BOUND_EXACT) {
    path = classify(head_slack(a.scale, head_max, bh));
    // Mode 4 never rounds Q.  Nor does a kernel with no bound loop to hand
    // the item to (the online-only persistent kernel, NODECLINE): in mode 1
    // it runs only when no head takes the bound loop, and should one still
    // test so, it keeps Q exact rather than leave the item undone.
    if ((a.mode == ATTN_SOFTMAX_BOUND_EXACT || NODECLINE) && path == kPre) path = kExact;
  }
  if (!per_tile && (path == kPre) != BOUND) return kDeclined;

  // Tile-wide max key norm over every attended 16-key granule.
  float km = 0.0f;
  if (BOUND || per_tile || path == kExact) {
    float* red = reinterpret_cast<float*>(smem + C::STAGE);
    const cf32* kg = k_gmax + (int64_t)bh * (a.N / 16);
    for (int e = e0; e < e1; ++e) {
      const int ks = kv_iv[2 * e], kl = kv_iv[2 * e + 1];
      if (!interval_ok(ks, kl, a.N)) continue;
      for (int g = ks / 16 + tid; g < (ks + kl) / 16; g += C::NT) km = fmaxf(km, kg[g]);
    }
    float qm = 0.0f;
    if (per_tile)
      for (int r = tid; r < nr; r += C::NT) qm = fmaxf(qm, q_norm[(int64_t)bh * a.N + qs + r]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      km = fmaxf(km, __shfl_xor(km, m));
      qm = fmaxf(qm, __shfl_xor(qm, m));
    }
    if (lane == 0) { red[wave] = km; red[NW + wave] = qm; }
    __syncthreads();
    km = red[0];
    qm = red[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) { km = fmaxf(km, red[i]); qm = fmaxf(qm, red[NW + i]); }
    // the same in every lane: keep them in scalar registers
    km = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, km)));
    qm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, qm)));
    if (per_tile) path = classify(2.0f * a.scale * qm * km);
    // `red` lies in a stage buffer that the first copies below overwrite:
    // every wave has to have read it first
    __syncthreads();
  }
  if (force_online) path = kOnline;
  if ((path == kPre) != BOUND) return kDeclined;
  const bool fixed = !BOUND && (path == kExact || path == kCheck);
  // (a checked tile whose check fails runs again at once, on the running
  // max, and overwrites this)
  if (tile == 0 && tid == 0 && a.head_path_out)
    a.head_path_out[bh] = path != kOnline ? ATTN_PATH_BOUND : ATTN_PATH_ONLINE;
  const float kfac = (BOUND || fixed) ? a.scale * km * kBoundMargin : 0.0f;

  Tile<D, NQB, NW, BOUND> T;
  T.fixed = __builtin_amdgcn_readfirstlane(fixed ? 1 : 0) != 0;
  T.n = lane & 31;
  T.hh = lane >> 5;
  T.lane = lane;
  T.lof = lane_offsets<D>(lane);
  T.set_addresses();
  // A tile of at most 64 rows runs thin (see run_thin): waves 4g to 4g+3
  // all hold row group g.
  bool thin = false;
  if constexpr (NQB == 1 && NW == 8 && !MASK) thin = nr <= 64;
  const int row0 = thin ? (wave >> 2) * 32 : wave * 32 * NQB;
  const u16* qh = a.q + b * a.sq[0] + h * a.sq[1];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = row0 + qb * 32 + T.n;
    const bool valid = r < nr;
    const u16* qp = qh + (int64_t)(qs + (valid ? r : 0)) * a.sq[2];
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st) {
      bf16x8 z = {};
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 16 * st + 8 * T.hh);
      if constexpr (BOUND) {
        // bound path: Q * scale * log2(e), rounded to bf16 (nearest even)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          f32x2 f = {(float)x[e] * a.c2, (float)x[e + 1] * a.c2};
          const bf16x2 b2 = __builtin_convertvector(f, bf16x2);
          x[e] = b2[0];
          x[e + 1] = b2[1];
        }
      }
      T.qreg[qb][st] = valid ? x : z;
    }
    if (BOUND || T.fixed) {
      const float qn = q_norm[(int64_t)bh * a.N + qs + (valid ? r : 0)];
      T.m2[qb] = valid ? qn * kfac * kLog2e : 0.0f;
      if constexpr (CHECK) {
        if (path == kCheck) T.m2[qb] -= kCheckShift2;
      }
    } else {
      T.m2[qb] = -INFINITY;
    }
    T.lsum[qb] = 0.0f;
    T.lsum2[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) T.oacc[qb][db][r2] = 0.0f;
  }

  const u16* kh = a.k + b * a.sk[0] + h * a.sk[1];
  const u16* vh = a.v + b * a.sv[0] + h * a.sv[1];
  // the upper half of the waves runs the lagging order (see run_tile)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // A wave none of whose rows exist (the short last tile of a frame) keeps
  // its share of the loads and barriers but skips the math.
  const bool active = thin ? wv < 4 * ((nr + 31) >> 5) : wv * 32 * NQB < nr;
  if constexpr (MASK) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) T.fq[qb] = (qs + min(row0 + qb * 32 + T.n, nr - 1)) / a.frame_T;
  }
  if (thin) {
    run_thin<D, NQB, NW, BOUND>(a, kv_iv, smem, T, kh, vh, e0, e1, wv, active);
  } else if (wv >= NW / 2) {
    run_tile<D, NQB, NW, BOUND, true, MASK>(a, kv_iv, smem, T, kh, vh, e0, e1, wv, active);
  } else {
    run_tile<D, NQB, NW, BOUND, false, MASK>(a, kv_iv, smem, T, kh, vh, e0, e1, wv, active);
  }
  if constexpr (CHECK && !BOUND) {
    // Mode 5 checks every tile that ran with a fixed shift (kExact or
    // kCheck; a kExact tile always passes, its certificate keeps l above
    // e^-ATTN_ELIGIBLE_NATS).  Both conditions are re-read rather than kept
    // in a register across the walk.  A row passes when its l is at least
    // 2^ATTN_CHECK_LOG2_L and finite and its accumulator finite (a kCheck
    // shift lies below the bound, so terms up to e^ATTN_CHECK_SHIFT_NATS
    // occur).
    if (T.fixed && a.mode == ATTN_SOFTMAX_BOUND_CHECKED) {
      // Every row's full l (both lane halves; after a thin walk, held by the
      // first wave of each row group) against 2^ATTN_CHECK_LOG2_L.
      bool low = false;
      if (active && (!thin || (wv & 3) == 0)) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float lh = T.lsum[qb] + T.lsum2[qb];
          const float lt = lh + __shfl_xor(lh, 32);
          bool ok = lt >= kCheckMinL && lt <= FLT_MAX;
#pragma unroll
          for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(T.oacc[qb][db][r]);
          low |= row0 + qb * 32 + T.n < nr && !ok;
        }
      }
      if (group_any<NW>(__any(low), smem, wv, lane)) return kRetry;
    }
  }
  if (thin && (wv & 3)) return kDone;  // merged into the first wave of the row group

  // Epilogue: O = O_acc / l (bf16, nearest even), LSE = m + ln l.
  u16* oh = a.o + b * a.so[0] + h * a.so[1];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lh = T.lsum[qb] + T.lsum2[qb];
    const float lt = lh + __shfl_xor(lh, 32);
    const int r = row0 + qb * 32 + T.n;
    if (r >= nr) continue;
    const float inv = 1.0f / lt;
    u16* op = oh + (int64_t)(qs + r) * a.so[2];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x2 f0 = {T.oacc[qb][db][4 * i] * inv, T.oacc[qb][db][4 * i + 1] * inv};
        f32x2 f1 = {T.oacc[qb][db][4 * i + 2] * inv, T.oacc[qb][db][4 * i + 3] * inv};
        bf16x2 b0 = __builtin_convertvector(f0, bf16x2), b1 = __builtin_convertvector(f1, bf16x2);
        u32x2 pk = {__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1)};
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * i + 4 * T.hh) = pk;
      }
    }
    if (T.hh == 0) {
      const int64_t ri = (int64_t)bh * a.N + qs + r;
      if (a.lse) a.lse[ri] = (T.m2[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
      if (a.shift_out) a.shift_out[ri] = T.m2[qb] * kLn2;
    }
  }
  return kDone;
}

// Static launch: workgroup i takes item work_order[i] (or i) on the path
// BOUND.  Both paths are launched over the same work; a workgroup whose item
// takes the other path exits at once, so each item is computed by exactly one
// of them and each path gets a register allocation of its own.
template <int D, int NQB, int NW, bool BOUND, bool MASK, bool CHECK>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(FwdArgs a, const int32_t* __restrict__ q_tiles,
                                                      const int32_t* __restrict__ kv_ptr,
                                                      const int32_t* __restrict__ kv_iv,
                                                      const int32_t* __restrict__ work_order,
                                                      const float* __restrict__ k_gmax,
                                                      const float* __restrict__ head_max) {
  using C = Cfg<D, NQB, NW>;
  __shared__ __attribute__((aligned(16))) u16 smem[kBuffers * C::STAGE];
  int w = blockIdx.x;
  if (work_order) {
    if (w >= a.n_work) return;
    w = work_order[w];
  }
  // a checked tile whose check failed runs again, on the running max
  for (bool force = false;; force = true) {
    const int r = run_item<D, NQB, NW, BOUND, MASK, CHECK>(a, (const ci32*)q_tiles, (const ci32*)kv_ptr,
                                                           (const ci32*)kv_iv, (const cf32*)k_gmax,
                                                           (const cf32*)head_max, smem, w, force);
    if (!CHECK || r != kRetry) break;
  }
}

// The kernel-argument segment (constant address space: scalar loads that no
// store of the kernel can alias).
typedef __attribute__((address_space(4))) const char kernarg_char;
typedef __attribute__((address_space(4))) const FwdArgs kernarg_args;

// A copy of the kernel arguments read through a pointer to the argument
// segment that the compiler cannot see through, so that two copies are two
// sets of loads rather than one set of values kept live between them.
// (`a`, the only kernel argument of fwd_persistent, starts the segment.)
__device__ __forceinline__ void item_args(FwdArgs& ia) {
  const kernarg_char* args = (const kernarg_char*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(args));
  static_assert(sizeof(FwdArgs) % 4 == 0, "FwdArgs is copied in dwords");
  typedef __attribute__((address_space(4))) const uint32_t kernarg_u32;
  const kernarg_u32* src = (const kernarg_u32*)args;
  uint32_t* dst = reinterpret_cast<uint32_t*>(&ia);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(FwdArgs) / 4); ++i) dst[i] = src[i];
}

// Persistent launch: one workgroup per CU, each taking items until none is
// left.  work_order holds n_xcd queues (slot j of queue x at j * n_xcd + x,
// padding -1 only at a queue's end); work_ctr[x] counts the slots of queue x
// handed out.  A workgroup takes slots from the queue of its own accelerator
// die (XCC) first -- the schedule keeps the tiles of one frame, which read
// the same keys, in one queue -- and then from the others, so a die that runs
// faster takes over work a slower one has not reached instead of idling
// while it finishes.  With BOTH, each item runs on its own softmax path in
// the same queue: the bound path's code takes it first and declines it,
// having written nothing, when the item takes the online path, which then
// runs it.  So online items (whole heads in mode 1, single tiles in mode 3)
// fill the same CUs as the bound ones instead of following them in a launch
// of their own.  Without BOTH the kernel holds the online path alone (modes
// 0 and 4, and in mode 1 the gated launch before the combined kernel):
// sharing a kernel with the bound path costs the online loop a few per
// cent.  The outputs do not depend on which workgroup computes an item.
template <int D, int NQB, int NW, bool MASK, bool BOTH, bool CHECK>
__global__ __launch_bounds__(64 * NW) void fwd_persistent(FwdArgs a) {
  (void)a;  // read through the argument-segment pointer below
  using C = Cfg<D, NQB, NW>;
  // The stage buffers, then 16 bytes that hold the item index: no stage copy
  // reaches them, so a workgroup can read its item again without keeping it
  // in a register.  (One LDS array: a separate LDS variable would cost the
  // operand reads their overlap with the stage copies, see tile_max.)
  __shared__ __attribute__((aligned(16))) u16 smem[kBuffers * C::STAGE + 8];
  // [0]: the item index; [1] (CHECK): 1 while the item is to run again.
  int32_t* const item_word = reinterpret_cast<int32_t*>(smem + kBuffers * C::STAGE);
  uint32_t empty = 0;  // thread 0: the queues found exhausted
  if constexpr (!BOTH) {
    // Gated (mode 1, launched before the combined kernel): when some head
    // takes the bound loop, leave every item to the combined kernel,
    // touching nothing.  Every wave tests every head (one per lane), so all
    // reach the same answer without a barrier.
    const kernarg_char* args = (const kernarg_char*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(args));
    const kernarg_args& ka = *reinterpret_cast<const kernarg_args*>(args);
    if (ka.gate == kGateOnline) {
      const cf32* hm = (const cf32*)ka.head_max;
      bool bound = false;
      for (int bh = threadIdx.x & 63; bh < ka.B * ka.H; bh += 64)
        bound |= head_slack(ka.scale, hm, bh) <= ATTN_PRESCALE_NATS;
      if (__any(bound)) return;
    }
  }
  if constexpr (CHECK) {
    if (threadIdx.x == 0) item_word[1] = 0;  // (read after the loop's first barrier)
  }
  for (;;) {
    __syncthreads();  // every wave is done with the previous item and has read its index
    // A checked tile whose check failed (run_item returned kRetry, in every
    // wave) runs again, on the running max: its index stays, and the flag
    // that says so is kept in LDS rather than in a register across the walk.
    const bool again = CHECK && __builtin_amdgcn_readfirstlane(item_word[1]) != 0;
    if (!again && threadIdx.x == 0) {
      // The queue layout and pointers are read here, through a pointer to
      // the kernel arguments the compiler cannot see through, rather than
      // held in scalar registers across the item (the walk needs them all).
      // (`a`, the only kernel argument, starts the segment)
      const kernarg_char* args = (const kernarg_char*)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(args));
      const kernarg_args& ka = *reinterpret_cast<const kernarg_args*>(args);
      const ci32* order = (const ci32*)ka.work_order;
      int32_t* counters = ka.work_ctr;
      const int nx = ka.n_xcd, depth = ka.n_work / nx;
      const int mine = (int)(__builtin_amdgcn_s_getreg(kHwRegXccId) & 0xF) % nx;
      int w = -1;
      for (int k = 0; k < nx && w < 0; ++k) {
        const int x = (mine + k) % nx;
        if ((empty >> x) & 1) continue;
        const int slot = atomicAdd(counters + x, 1);
        const int cand = slot < depth ? order[slot * nx + x] : -1;
        if (cand < 0) empty |= 1u << x;
        else w = cand;
      }
      item_word[0] = w;
    }
    __syncthreads();
    const int w = __builtin_amdgcn_readfirstlane(item_word[0]);
    if (w < 0) break;
    // Each path reads the item's arguments afresh through the opaque
    // pointer, so none is held in a scalar register from one item, or one
    // path, to the next.  (a declined item has finished with the LDS it
    // used: see run_item)
    bool done = false;
    if constexpr (BOTH) {
      if (!again) {
        FwdArgs ia;
        item_args(ia);
        done = run_item<D, NQB, NW, true, MASK, CHECK>(ia, (const ci32*)ia.q_tiles, (const ci32*)ia.kv_ptr,
                                                       (const ci32*)ia.kv_iv, (const cf32*)ia.k_gmax,
                                                       (const cf32*)ia.head_max, smem, w) != kDeclined;
      }
    }
    if (!done) {
      FwdArgs ib;
      item_args(ib);
      const bool force = CHECK && __builtin_amdgcn_readfirstlane(item_word[1]) != 0;
      const int r = run_item<D, NQB, NW, false, MASK, CHECK, !BOTH>(
          ib, (const ci32*)ib.q_tiles, (const ci32*)ib.kv_ptr, (const ci32*)ib.kv_iv, (const cf32*)ib.k_gmax,
          (const cf32*)ib.head_max, smem, w, force);
      if constexpr (CHECK) {
        // (both cases walked the tile, past barriers that follow every
        // wave's reads of the flag)
        if (threadIdx.x == 0 && (r == kRetry || force)) item_word[1] = r == kRetry ? 1 : 0;
      }
    }
  }
  // Leaving: work_ctr[n_xcd] counts the workgroups that are done.  The last
  // one (every other workgroup has made its last slot request, as it counts
  // itself only after them) sets all counters back to zero for the next call
  // on this workspace -- or, after a gated online-only launch that ran the
  // items, every queue counter to its depth: the combined kernel launched
  // next then finds every queue exhausted, and its last workgroup zeroes them.
  if (threadIdx.x == 0) {
    const kernarg_char* args = (const kernarg_char*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(args));
    const kernarg_args& ka = *reinterpret_cast<const kernarg_args*>(args);
    int32_t* counters = ka.work_ctr;
    const int nx = ka.n_xcd;
    const int left = !BOTH && ka.gate == kGateOnline ? ka.n_work / nx : 0;
    // (atomic writes: the next call's slot requests may come from other dies)
    if (atomicAdd(counters + nx, 1) == (int)gridDim.x - 1)
      for (int x = 0; x <= nx; ++x) atomicExch(counters + x, x < nx ? left : 0);
  }
}


static_assert(ONLINE_NQB == BOUND_NQB && ONLINE_NW == BOUND_NW,
              "the persistent kernel runs both paths on one tile shape");

template <int D, int NQB, int NW, bool MASK>
int launch_persistent(const FwdArgs& a, int grid, bool both, bool check, hipStream_t stream) {
  if constexpr (!MASK) {  // (the frame-unaware layout does not take mode 5)
    if (check) {
      hipLaunchKernelGGL((fwd_persistent<D, NQB, NW, MASK, true, true>), dim3(grid), dim3(64 * NW), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
      return ok();
    }
  }
  if (both && a.mode == ATTN_SOFTMAX_BOUND) {
    // Per-head mode: when no head takes the bound loop, the online-only
    // kernel runs every item (the online loop of the combined kernel runs a
    // few per cent slower) and leaves the queues exhausted for the combined
    // kernel; otherwise it leaves at once and the combined kernel runs them.
    FwdArgs g = a;
    g.gate = kGateOnline;
    hipLaunchKernelGGL((fwd_persistent<D, NQB, NW, MASK, false, false>), dim3(grid), dim3(64 * NW), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    hipLaunchKernelGGL((fwd_persistent<D, NQB, NW, MASK, true, false>), dim3(grid), dim3(64 * NW), 0, stream, a);
  } else if (both) {
    hipLaunchKernelGGL((fwd_persistent<D, NQB, NW, MASK, true, false>), dim3(grid), dim3(64 * NW), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fwd_persistent<D, NQB, NW, MASK, false, false>), dim3(grid), dim3(64 * NW), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return ok();
}

template <int D, int NQB, int NW, bool BOUND, bool MASK>
int launch(const FwdArgs& a, int grid, bool check, hipStream_t stream) {
  if constexpr (!BOUND && !MASK) {  // (the frame-unaware layout does not take mode 5)
    if (check) {
      hipLaunchKernelGGL((fwd_kernel<D, NQB, NW, BOUND, MASK, true>), dim3(grid), dim3(64 * NW), 0, stream, a,
                         a.q_tiles, a.kv_ptr, a.kv_iv, a.work_order, a.k_gmax, a.head_max);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
      return ok();
    }
  }
  hipLaunchKernelGGL((fwd_kernel<D, NQB, NW, BOUND, MASK, false>), dim3(grid), dim3(64 * NW), 0, stream, a,
                     a.q_tiles, a.kv_ptr, a.kv_iv, a.work_order, a.k_gmax, a.head_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return ok();
}

// Sets n counters to zero (vector stores), before a persistent launch that
// takes its slot counters from the library's own array (attn_fwd_noalloc).
__global__ __launch_bounds__(64) void zero_counters(int32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

}  // namespace
}  // namespace bsvf

// The slot counters of attn_fwd_noalloc's persistent launch: a fixed array
// in device memory, one copy per GPU, held until the process ends.  Host
// code never names it as an address: each device's copy is found once with
// hipGetSymbolAddress (noalloc_counters below) and passed to the kernels.
static __device__ __align__(256) int32_t scratch[64];
static_assert(ATTN_NOALLOC_MAX_XCD + 1 <= 64, "scratch holds the counters of up to ATTN_NOALLOC_MAX_XCD queues");

namespace bsvf {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int noalloc_counters(int32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ATTN_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_E_UNSUPPORTED, "attn_fwd_noalloc supports device indices below 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ATTN_E_HIP, std::string("hipGetSymbolAddress of the counter array failed: ") + hipGetErrorString(e));
    g_scratch[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch[dev];
  return ok();
}

}  // namespace
}  // namespace bsvf

using namespace bsvf;

static int fwd_entry(const void* q, const void* k, const void* v, void* o, float* lse, float* shift_out,
                     int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim, const int64_t* strides,
                     float scale, const attn_blocks_t* blocks, const int32_t* kv_flag,
                     const attn_pattern_t* pattern, const float* q_norm, const float* k_gmax,
                     const float* head_max, int32_t softmax_mode, int32_t* head_path_out, hipStream_t stream,
                     bool noalloc = false) {
  const bool masked = pattern != nullptr;
  if (batch <= 0 || heads <= 0 || seq_len <= 0) return fail(ATTN_E_INVAL, "sizes must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(ATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (seq_len % 16) return fail(ATTN_E_ALIGN, "seq_len must be a multiple of 16");
  if (!strides) return fail(ATTN_E_INVAL, "strides is NULL");
  if (!(scale > 0.0f) || !(scale < 3.0e38f)) return fail(ATTN_E_INVAL, "scale must be positive and finite");
  if (softmax_mode < ATTN_SOFTMAX_ONLINE || softmax_mode > ATTN_SOFTMAX_BOUND_CHECKED)
    return fail(ATTN_E_INVAL, "bad softmax_mode");
  if (masked && softmax_mode == ATTN_SOFTMAX_BOUND_CHECKED)
    return fail(ATTN_E_UNSUPPORTED, "the frame-unaware layout takes softmax modes 0 to 4");
  int st;
  if ((st = check_tensor("q", q, strides + 0, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("k", k, strides + 3, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("v", v, strides + 6, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("o", o, strides + 9, batch, heads, seq_len, head_dim))) return st;
  if (!blocks) return fail(ATTN_E_INVAL, "blocks is NULL");
  if (!blocks->q_tiles || !blocks->kv_ptr || !blocks->kv_iv) return fail(ATTN_E_INVAL, "block list pointers are NULL");
  if (blocks->n_qt <= 0 || blocks->nnz <= 0) return fail(ATTN_E_INVAL, "n_qt and nnz must be positive");
  if (blocks->block_q <= 0 || blocks->block_q % 16) return fail(ATTN_E_ALIGN, "block_q must be a positive multiple of 16");
  if (blocks->block_q > ATTN_MAX_BLOCK_Q) return fail(ATTN_E_UNSUPPORTED, "block_q exceeds ATTN_MAX_BLOCK_Q");
  if (blocks->work_order && blocks->n_work <= 0) return fail(ATTN_E_INVAL, "n_work must be positive");
  if (softmax_mode != ATTN_SOFTMAX_ONLINE && (!q_norm || !k_gmax || !head_max))
    return fail(ATTN_E_UNSUPPORTED, "bound softmax needs q_norm, k_gmax and head_max");
  uint64_t gbits = 0;
  if (masked) {
    if (!kv_flag) return fail(ATTN_E_INVAL, "kv_flag is NULL");
    if (pattern->tokens_per_frame < 64) return fail(ATTN_E_UNSUPPORTED, "the frame mask needs tokens_per_frame >= 64");
    if ((int64_t)pattern->num_frames * pattern->tokens_per_frame != seq_len)
      return fail(ATTN_E_PATTERN, "num_frames * tokens_per_frame must equal seq_len");
    if (pattern->win_before < 0 || pattern->win_after < 0) return fail(ATTN_E_PATTERN, "windows must be >= 0");
    if (pattern->num_global < 0 || (pattern->num_global > 0 && !pattern->global_frames))
      return fail(ATTN_E_INVAL, "bad global frame list");
    for (int32_t i = 0; i < pattern->num_global; ++i) {
      const int32_t g = pattern->global_frames[i];
      if (g < 0 || g >= pattern->num_frames) return fail(ATTN_E_PATTERN, "global frame out of range");
      if (g >= 64) return fail(ATTN_E_UNSUPPORTED, "global frames must be below 64");
      gbits |= (uint64_t)1 << g;
    }
  }
  const int64_t items = (int64_t)blocks->n_qt * heads * batch;
  if (items > 2147483647LL) return fail(ATTN_E_SIZE, "too many work items");
  if ((int64_t)batch * heads * seq_len > 2147483647LL) return fail(ATTN_E_SIZE, "B*H*N exceeds INT32_MAX");

  FwdArgs a;
  a.q = static_cast<const u16*>(q);
  a.k = static_cast<const u16*>(k);
  a.v = static_cast<const u16*>(v);
  a.o = static_cast<u16*>(o);
  a.lse = lse;
  a.shift_out = shift_out;
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = strides[i];
    a.sk[i] = strides[3 + i];
    a.sv[i] = strides[6 + i];
    a.so[i] = strides[9 + i];
  }
  a.B = batch;
  a.H = heads;
  a.N = seq_len;
  a.scale = scale;
  a.c2 = scale * kLog2e;
  a.q_tiles = blocks->q_tiles;
  a.kv_ptr = blocks->kv_ptr;
  a.kv_iv = blocks->kv_iv;
  a.n_qt = blocks->n_qt;
  a.nnz = blocks->nnz;
  a.block_q = blocks->block_q;
  a.work_order = blocks->work_order;
  a.n_work = blocks->work_order ? blocks->n_work : 0;
  a.q_norm = q_norm;
  a.k_gmax = k_gmax;
  a.head_max = head_max;
  a.mode = softmax_mode;
  a.gate = kGateNone;
  const bool check = softmax_mode == ATTN_SOFTMAX_BOUND_CHECKED;
  a.head_path_out = head_path_out;
  a.kv_flag = kv_flag;
  a.frame_T = masked ? pattern->tokens_per_frame : 0;
  a.win_lo = masked ? -pattern->win_before : 0;
  a.win_hi = masked ? pattern->win_after : 0;
  a.gbits[0] = (uint32_t)gbits;
  a.gbits[1] = (uint32_t)(gbits >> 32);

  if (blocks->work_ctr) {
    if (noalloc) return fail(ATTN_E_INVAL, "attn_fwd_noalloc keeps its counters itself: blocks->work_ctr must be NULL");
    if (!blocks->work_order) return fail(ATTN_E_INVAL, "work_ctr needs a work_order");
    if (blocks->num_xcd < 1 || blocks->num_xcd > 32) return fail(ATTN_E_INVAL, "num_xcd must be in [1, 32]");
    if (blocks->n_work % blocks->num_xcd) return fail(ATTN_E_INVAL, "n_work must be a multiple of num_xcd");
  }
  if (noalloc) {
    if (!blocks->work_order) return fail(ATTN_E_INVAL, "attn_fwd_noalloc needs a work_order (from attn_build_schedule)");
    if (blocks->num_xcd < 1) return fail(ATTN_E_INVAL, "num_xcd must be at least 1");
    if (blocks->num_xcd > ATTN_NOALLOC_MAX_XCD)
      return fail(ATTN_E_SIZE, "attn_fwd_noalloc holds counters for at most ATTN_NOALLOC_MAX_XCD (32) queues");
    if (blocks->n_work % blocks->num_xcd) return fail(ATTN_E_INVAL, "n_work must be a multiple of num_xcd");
  }
  int32_t* ctr = blocks->work_ctr;
  if (noalloc && (st = noalloc_counters(&ctr))) return st;
  a.n_xcd = ctr ? blocks->num_xcd : 1;
  a.work_ctr = ctr;
  const int grid = blocks->work_order ? blocks->n_work : (int)items;
  const int bq_bound = 32 * BOUND_NQB * BOUND_NW, bq_online = 32 * ONLINE_NQB * ONLINE_NW;
  if (blocks->block_q > (softmax_mode == ATTN_SOFTMAX_BOUND_FORCED ? bq_bound
                         : softmax_mode == ATTN_SOFTMAX_ONLINE ? bq_online : min(bq_bound, bq_online)))
    return fail(ATTN_E_UNSUPPORTED, "block_q exceeds the kernels' query tile of 256 rows");
  // With a work_ctr, one persistent launch runs every item on its path (one
  // workgroup per CU; a workgroup takes most of a CU's LDS); in the modes
  // without the prescaled Q (0 and 4) its kernel holds the online loop only.
  // Without one, each path has a launch of one workgroup per item.
  int cus = 0;
  if (ctr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return fail(ATTN_E_HIP, "cannot query the number of compute units");
  }
  if (cus > 0) {
    const int pgrid = std::min(blocks->n_work, cus);
    // the bound loop is needed unless every item runs on the online loop
    const bool both = softmax_mode != ATTN_SOFTMAX_ONLINE && softmax_mode != ATTN_SOFTMAX_BOUND_EXACT;
    // mode 5 has kernels of its own: only they hold the check and the retry
    if (noalloc) {
      // the shared array keeps the last call's contents: start from zero
      hipLaunchKernelGGL(zero_counters, dim3(1), dim3(64), 0, stream, ctr, blocks->num_xcd + 1);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    }
    if (masked)
      st = head_dim == 128 ? launch_persistent<128, BOUND_NQB, BOUND_NW, true>(a, pgrid, both, check, stream)
                           : launch_persistent<64, BOUND_NQB, BOUND_NW, true>(a, pgrid, both, check, stream);
    else
      st = head_dim == 128 ? launch_persistent<128, BOUND_NQB, BOUND_NW, false>(a, pgrid, both, check, stream)
                           : launch_persistent<64, BOUND_NQB, BOUND_NW, false>(a, pgrid, both, check, stream);
    return st ? st : ok();
  }
  if (softmax_mode != ATTN_SOFTMAX_ONLINE && softmax_mode != ATTN_SOFTMAX_BOUND_EXACT) {
    if (masked)
      st = head_dim == 128 ? launch<128, BOUND_NQB, BOUND_NW, true, true>(a, grid, check, stream)
                           : launch<64, BOUND_NQB, BOUND_NW, true, true>(a, grid, check, stream);
    else
      st = head_dim == 128 ? launch<128, BOUND_NQB, BOUND_NW, true, false>(a, grid, check, stream)
                           : launch<64, BOUND_NQB, BOUND_NW, true, false>(a, grid, check, stream);
    if (st) return st;
  }
  if (softmax_mode != ATTN_SOFTMAX_BOUND_FORCED) {
    if (masked)
      st = head_dim == 128 ? launch<128, ONLINE_NQB, ONLINE_NW, false, true>(a, grid, check, stream)
                           : launch<64, ONLINE_NQB, ONLINE_NW, false, true>(a, grid, check, stream);
    else
      st = head_dim == 128 ? launch<128, ONLINE_NQB, ONLINE_NW, false, false>(a, grid, check, stream)
                           : launch<64, ONLINE_NQB, ONLINE_NW, false, false>(a, grid, check, stream);
    if (st) return st;
  }
  return ok();
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
                        int32_t head_dim, const int64_t* strides, float scale,
                        const attn_blocks_t* blocks, const float* q_norm, const float* k_gmax,
                        const float* head_max, int32_t softmax_mode, int32_t* head_path_out,
                        hipStream_t stream) {
  return fwd_entry(q, k, v, o, lse, shift_out, batch, heads, seq_len, head_dim, strides, scale, blocks,
                   nullptr, nullptr, q_norm, k_gmax, head_max, softmax_mode, head_path_out, stream);
}

extern "C" int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
                                int32_t head_dim, const int64_t* strides, float scale,
                                const attn_blocks_t* blocks, const float* q_norm, const float* k_gmax,
                                const float* head_max, int32_t softmax_mode, int32_t* head_path_out,
                                hipStream_t stream) {
  return fwd_entry(q, k, v, o, lse, shift_out, batch, heads, seq_len, head_dim, strides, scale, blocks,
                   nullptr, nullptr, q_norm, k_gmax, head_max, softmax_mode, head_path_out, stream, true);
}

extern "C" int attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                               float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
                               int32_t head_dim, const int64_t* strides, float scale,
                               const attn_blocks_t* blocks, const int32_t* kv_flag,
                               const attn_pattern_t* pattern, const float* q_norm,
                               const float* k_gmax, const float* head_max, int32_t softmax_mode,
                               int32_t* head_path_out, hipStream_t stream) {
  if (!pattern) return fail(ATTN_E_INVAL, "pattern is NULL");
  return fwd_entry(q, k, v, o, lse, shift_out, batch, heads, seq_len, head_dim, strides, scale, blocks,
                   kv_flag, pattern, q_norm, k_gmax, head_max, softmax_mode, head_path_out, stream);
}
