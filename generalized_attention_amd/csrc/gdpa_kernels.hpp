// Kernel argument blocks and host-side launchers of the GDPA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdpa {

// Activation kinds after folding the enum aliases (FAST_GELU*, GELU_TANH -> GELU_TANH;
// FAST_SILU -> SILU).  Values match gdpa_act_t.
// Element types of the MFMA inputs: bf16 or fp16 Q, K, V (and dO), or FP8
// E4M3 Q and K with bf16 V (forward only).
// EL_MX8: MXFP8 (E4M3, E8M0 scale per 32); EL_MX4: MXFP4 (E2M1 pairs per byte, E8M0 scale per 32)
enum ElemKind : int { EL_BF16 = 0, EL_F16 = 1, EL_FP8 = 2, EL_MX8 = 3, EL_MX4 = 4 };
// Output element types.
enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

enum ActKind : int {
  ACT_IDENTITY = 0,
  ACT_GELU = 1,
  ACT_GELU_TANH = 2,
  ACT_RELU = 5,
  ACT_RELU2 = 6,
  ACT_LEAKY = 7,
  ACT_SILU = 8,
  ACT_HARDSWISH = 10,
};


// Activation constants with the score scale folded in (computed on the host).
// With c = scale (times the FP8 descales) and s the raw dot product q.k, the
// kernels evaluate y(s) such that act(c s) = pscale * y(s), and d(s) =
// act'(c s); the chain-rule factor c of dQ and dK is applied once, as gscale,
// to the accumulators.  k0, k1, a0, a1 are per-activation (see gdpa_common.hpp).
struct ActConsts {
  float k0, k1, a0, a1;
  float alpha;    // LeakyReLU slope
  float pscale;   // act(c s) = pscale * y(s)
  float gscale;   // = c
};

// One forward launch.  Sequence b of a jagged batch owns query rows
// cu_q[b]..cu_q[b+1]-1 and key rows cu_k[b]..cu_k[b+1]-1; with cu_q == nullptr
// the batch is fixed-length (lq_fixed / lk_fixed rows per sequence).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t lq_fixed;
  int32_t lk_fixed;
  int32_t hq;
  int32_t hkv;
  int32_t group;      // hq / hkv
  int32_t mblocks;    // ceil(max_seqlen_q / 128)
  ActConsts act;      // activation constants (c = scale * q_descale * k_descale)
  int32_t wl;         // window left  (-1: unbounded)
  int32_t wr;         // window right (-1: unbounded)
  int32_t out_kind;   // OUT_F32, OUT_BF16 or OUT_F16
  int32_t psplit;     // 1: P carried as a 16-bit hi/lo pair (two MFMAs for P V)
  const int32_t* perm;  // sequences in processing order (costliest first), or nullptr
  const uint8_t* q_mx;  // MXFP8: E8M0 scales of q [total_q, Hq, D / 32] (else nullptr)
  const uint8_t* k_mx;  //        and of k [total_k, Hkv, D / 32]
};

// One backward launch (both kernels take the same block).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t lq_fixed;
  int32_t lk_fixed;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t mblocks;    // dQ kernel: ceil(max_seqlen_q / 128)
  int32_t nblocks;    // dK/dV kernel: ceil(max_seqlen_k / 128)
  ActConsts act;      // activation constants (c = scale)
  int32_t wl;
  int32_t wr;
  int32_t out_kind;   // OUT_F32, OUT_BF16 or OUT_F16 (dQ, dK, dV)
  int32_t dsplit;     // 1: dS carried as a 16-bit hi/lo pair in dQ = dS K
  int32_t kvsplit;    // 1: P and dS carried as 16-bit hi/lo pairs in dV, dK
  const int32_t* perm;  // sequences in processing order (costliest first), or nullptr
  int32_t* counters;    // per-XCD dK/dV work-queue counters (zeroed by the schedule), or nullptr
  int32_t ncu;          // compute units of the device (sizes the work-queue launches)
  // Fused backward (dQ accumulated inside the dK/dV kernel), all zeroed by
  // the call before the kernel runs:
  float* dq_acc;        // fp32 dQ accumulator [total_q, hq, D] (dq itself when dQ is fp32)
  int32_t* turn;        // per (64-row query tile, query head) turn counters
  int32_t* qstate;      // per queue: next item [8], owning XCD + 1 [8]; then the error flag
  int32_t mt_fixed;     // fixed-length batches: 64-row query tiles per sequence
  int32_t spin_limit;   // polls before a turn wait gives up and sets the error flag
  // factors of the dQ and dK stores: the chain-rule factor c (act.gscale),
  // divided by the per-tensor scale that S folds in but the other operand
  // of the product does not carry (FP8 Q/K codes; 1 otherwise)
  float dq_scale;
  float dk_scale;
};

// Forward workgroup: kFwdNW waves, each owning 32 query rows.
constexpr int kFwdNW = 4;
constexpr int kFwdBM = 32 * kFwdNW;
// XCDs per MI355X; workgroup ids are dealt to them round-robin.
constexpr int kNumXcd = 8;

// Workgroup -> work item.  Work is grouped by (sequence, KV head) pair; a
// pair owns per_pair consecutive items (query heads x query blocks, or key
// blocks).  The dispatcher deals consecutive workgroup ids to the XCDs in
// turn and each XCD has its own L2, so pair p goes to XCD p % 8 and all its
// items run there back to back: each K/V (or Q/dO) tile is fetched into that
// L2 once and re-read there by the pair's other workgroups.  Pairs are taken
// in rank order of perm (costliest sequences first, when a schedule was built),
// so every XCD works through its share costliest-first and short items fill the
// tail.  The grid is the pair count rounded up to the XCD count, times per_pair.
inline long pair_grid(long batch, long hkv, long per_pair) {
  const long pairs = ((long)batch * hkv + kNumXcd - 1) / kNumXcd * kNumXcd;
  return pairs * per_pair;
}
struct WorkItem {
  int b;     // sequence
  int g;     // KV head
  int rest;  // index within the pair, 0 .. per_pair-1
};
__device__ __forceinline__ bool map_work(int bid, int batch, int hkv, int per_pair, const int32_t* perm,
                                         WorkItem& w) {
  const int xcd = bid & (kNumXcd - 1), local = bid / kNumXcd;
  const int pair = (local / per_pair) * kNumXcd + xcd;
  if (pair >= batch * hkv) return false;
  const int rank = pair / hkv;
  w.b = perm != nullptr ? perm[rank] : rank;
  w.g = pair % hkv;
  w.rest = local % per_pair;
  return true;
}
inline long fwd_grid(const FwdArgs& a) { return pair_grid(a.batch, a.hkv, (long)a.group * a.mblocks); }

// Queue-mode grid: occ workgroups per CU, a multiple of the XCD count so that
// every XCD's queue has workgroups draining it.
inline long queue_grid(int ncu, int occ) {
  const long n = (long)ncu * occ;
  return n < kNumXcd ? kNumXcd : (n + kNumXcd - 1) / kNumXcd * kNumXcd;
}

// Queue mode: the pairs of this workgroup's XCD and the pair of its list entry j.
__device__ __forceinline__ long xcd_items(int batch, int hkv, int per_pair) {
  const int xcd = blockIdx.x & (kNumXcd - 1);
  const int pairs = batch * hkv;
  return pairs > xcd ? (long)((pairs - xcd + kNumXcd - 1) / kNumXcd) * per_pair : 0;
}
__device__ __forceinline__ void xcd_item(int j, int hkv, int per_pair, const int32_t* perm, WorkItem& w) {
  const int pair = (j / per_pair) * kNumXcd + (int)(blockIdx.x & (kNumXcd - 1));
  w.b = perm[pair / hkv];
  w.g = pair % hkv;
  w.rest = j % per_pair;
}

// Longest-first schedule of a jagged batch: perm[r] is the sequence with the
// r-th largest cost, the number of 64 x 64 (query, key) blocks in which the
// window (wl, wr) (-1 = unbounded side) leaves an allowed pair (ties by
// larger lq + lk, then by index).  Built on the device by one workgroup for
// batches of at most kSortMax sequences, which also zeroes kNumCounters
// work-queue counters; larger batches keep index order.
constexpr int kSortMax = 4096;
constexpr int kNumCounters = kNumXcd;

// Blocks of 64 queries x 64 keys that hold at least one allowed pair of a
// sequence with lq queries and lk keys under the window (wl, wr) (-1 =
// unbounded side; bottom-right aligned: query i sees keys i + lk - lq - wl ..
// i + lk - lq + wr).  Each 64-query tile's allowed keys form one interval,
// the union of its rows' intervals, which shift by one key per row.
__host__ __device__ inline int64_t mask_blocks(int lq, int lk, int wl, int wr) {
  if (lq <= 0 || lk <= 0) return 0;
  const int64_t mt = (lq + 63) / 64, nt = (lk + 63) / 64;
  if (wl < 0 && wr < 0) return mt * nt;
  const int64_t off = (int64_t)lk - lq;
  int64_t n = 0;
  for (int64_t t = 0; t < mt; ++t) {
    const int64_t r0 = 64 * t, r1 = r0 + 63 < lq - 1 ? r0 + 63 : lq - 1;
    const int64_t lo = wl < 0 ? 0 : (r0 + off - wl > 0 ? r0 + off - wl : 0);
    const int64_t hi = wr < 0 ? lk - 1 : (r1 + off + wr < lk - 1 ? r1 + off + wr : lk - 1);
    if (lo <= hi) n += hi / 64 - lo / 64 + 1;
  }
  return n;
}
// Sort key of sequence i: ascending keys run the larger cost first, then the
// larger lq + lk, then the smaller index, which the low 12 bits hold.
static_assert(kSortMax <= 4096, "the sort key keeps the sequence index in 12 bits");
__host__ __device__ inline uint64_t schedule_key(int lq, int lk, int wl, int wr, int i) {
  const int64_t cost = mask_blocks(lq, lk, wl, wr);
  const int64_t len = (int64_t)lq + lk;
  const uint64_t icost = (uint64_t)(0xffffffffLL - (cost < 0xffffffffLL ? cost : 0xffffffffLL));
  const uint64_t ilen = (uint64_t)(0xfffffLL - (len < 0xfffffLL ? len : 0xfffffLL));
  return (icost << 32) | (ilen << 12) | (uint64_t)(i & 0xfff);
}
__host__ __device__ inline int32_t schedule_key_index(uint64_t key) { return (int32_t)(key & 0xfffu); }
hipError_t launch_schedule(const int32_t* cu_q, const int32_t* cu_k, int batch, int wl, int wr, int32_t* perm,
                           int32_t* counters, hipStream_t stream);
// Zeroes n int32 words at p (a kernel, not a memset, so the call stays
// capturable in a graph).
hipError_t launch_zero(int32_t* p, long n, hipStream_t stream);
// Decodes rows of FP8 E4M3 codes (in_kind EL_FP8), MXFP8 (EL_MX8) or MXFP4
// (EL_MX4, two elements per byte) with their E8M0 block scales (MX kinds) to
// bf16: rows x d values (d a multiple of 32).  FP8 codes are written as their
// E4M3 values (the per-tensor scale stays with the caller).
hipError_t launch_decode_bf16(const uint8_t* src, const uint8_t* scales, uint16_t* dst, long rows, int d, int in_kind,
                              hipStream_t stream);

// Fused backward: queue state layout inside BwdArgs::qstate.
constexpr int kQNext = 0, kQOwner = kNumXcd, kQErr = 2 * kNumXcd, kQWords = 2 * kNumXcd + 1;
// Turn counters are indexed by (first tile of the sequence + tile) * hq + head
// with a sequence's first tile at cu_q[b] / 64 + b (jagged) or b * mt_fixed:
// fewer than total_q / 64 + batch tiles in all.
constexpr int kDqTile = 64;

// Work-queue execution (jagged batches with a schedule): a launch of as many
// workgroups as the device holds at once.  Work is still grouped by (sequence,
// KV head) pair with pair p on XCD p % 8 (L2 reuse of the pair's tiles), but
// the workgroups of an XCD take the next item of that XCD's list from an
// atomic counter instead of being handed one item each by the dispatcher.
// The lists run costliest sequence first, so a free workgroup always picks the
// heaviest remaining item of its XCD (list scheduling).  The next index is
// taken as the current item enters its last step (the body calls
// fetch.issue() there; the counter's reply arrives while the step computes):
// an index taken any earlier would reserve the heaviest remaining item for a
// workgroup that stays busy for longer, while workgroups that free up in the
// meantime take lighter ones, and the tail of the launch would lose the
// costliest-first order.  Workgroup ids are dealt to the XCDs in turn, so
// blockIdx % 8 names the XCD (only locality depends on that).
struct QueueFetch {
  int32_t* counter;
  int32_t* slot;  // LDS word that receives the next index
  int32_t v;
  __device__ __forceinline__ void issue() {
    if (threadIdx.x == 0) v = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void publish() {
    if (threadIdx.x == 0) *slot = v;
  }
};
template <typename F>
__device__ __forceinline__ void run_queue(int32_t* counter, long total, F&& body) {
  __shared__ int32_t nxt[2];
  if (threadIdx.x == 0) nxt[0] = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int item = nxt[0];
  int par = 0;
  while (item < total) {
    // the slot written during this item is read only after the barrier below;
    // the other slot was read before the previous one
    // body(item, fetch) calls fetch.issue() at most once and returns whether it did
    QueueFetch fetch{counter, &nxt[par ^ 1], 0};
    if (!body(item, fetch)) fetch.issue();
    fetch.publish();
    __syncthreads();
    item = nxt[par ^ 1];
    par ^= 1;
  }
}

// Backward: dK/dV blocks cover 128 key rows, dQ blocks 128 query rows.
constexpr int kBwdBN = 128;
constexpr int kBwdBM = 128;

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int head_dim_v, int act_kind, int in_kind, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int head_dim, int act_kind, int in_kind, bool want_dq, bool want_dkv,
                      bool fused, hipStream_t stream);
// fp16 forward instantiations (own translation unit)
hipError_t launch_fwd_f16(const FwdArgs& a, int head_dim, int head_dim_v, int act_kind, hipStream_t stream);

}  // namespace gdpa
