// Host layer of libmoe: argument checks, the capacity rule, workspace
// carving, path choice and the launch sequence of every entry point declared
// in include/moe.h.  No memory is allocated here; scratch comes from the
// caller's workspace.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// ----------------------------------------------------------------- timing
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};
struct TimingState {
  std::mutex mu;
  bool enabled = false;
  std::vector<std::string> only;   // groups to time; empty: all
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> free_events;
  std::vector<std::string> names;
  std::vector<int64_t> launches;
  std::vector<double> total_ms;
};
TimingState& timing() {
  static TimingState t;
  return t;
}

hipEvent_t take_event(TimingState& t) {
  if (!t.free_events.empty()) {
    hipEvent_t e = t.free_events.back();
    t.free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with events when timing is enabled.
class Timed {
 public:
  Timed(const char* name, hipStream_t s) : name_(name), s_(s) {
    TimingState& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (!t.enabled) return;
    if (!t.only.empty() &&
        std::find(t.only.begin(), t.only.end(), std::string(name)) == t.only.end())
      return;
    start_ = take_event(t);
    stop_ = take_event(t);
    if (start_ && stop_) hipEventRecord(start_, s_);
  }
  ~Timed() {
    if (!start_ || !stop_) return;
    hipEventRecord(stop_, s_);
    TimingState& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    t.pending.push_back(TimedLaunch{name_, start_, stop_});
  }

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// ----------------------------------------------------------------- plan
constexpr size_t kAlign = 256;

// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Region {
  size_t off = 0, bytes = 0;
};

// Debug canaries (moe_debug_canaries): with them on, every workspace region
// is followed by a guard of kCanaryBytes holding kCanaryByte, written at the
// start of each call and compared by moe_debug_check, so a kernel that
// writes past the end of its region is caught.
constexpr int kMaxGuards = 48;
constexpr size_t kCanaryBytes = 256;
constexpr unsigned char kCanaryByte = 0xA5;
std::atomic<bool> g_canaries{false};

struct Plan {
  int64_t T = 0;
  int d = 0, F = 0, E = 0, k = 0, S = 0;
  int gating = 0, renorm = 0;
  bool bf16 = false;
  int path = MOE_PATH_GROUPED;   // resolved
  int64_t capacity = 0;          // exact C
  int overflow = MOE_OVERFLOW_DROP;
  int Ceff = 0;                  // rows per expert the dispatch keeps: min(C, T),
                                 // or T when nothing is dropped (sequential)
  int64_t TK = 0;
  int64_t rows_max = 0;          // most kept rows possible
  int nblk_dispatch = 0;
  int topk_blocks = 0, topk_tpb = 0;
  int bm = 0;                    // M-tile of the grouped kernels
  int max_mtiles = 0;
  int static_bm = 0;             // M-tile of the GEMMs over all T token rows
  bool mfma_router = false;      // router scores on the MFMA GEMM (bf16, E % 8 == 0)
  bool parts_router = false;     // short batches: the K-part router instead
  bool narrow_router = false;    // few experts: the narrow MFMA router instead
  int router_split = 1;          // K parts of the router GEMM
  int ffn2_kcut_slots = 0;       // > 0: the routed down projection's two K parts cut for this many slots
  int ffn2_split = 1;            // K parts of the routed down projection
  int shared2_split = 1;         // K parts of the shared down projection
  bool small_route = false;      // top-k and dispatch in one workgroup
  bool blocked = false;          // GEMM1 writes H K-blocked; GEMM2 reads it so
  bool gather_x = false;         // GEMM1 reads a gathered, K-blocked copy of the token rows
  // workspace regions
  Region logits, lpart, idx, w, lrank, blkcnt, counts, kcount, offsets, slot, perm,
      tiles, ntiles, tstart, ppart, hpart, stats, H, Hs, Y, Ys, Xb, ovf, xdest, xrel, gpart,
      bdlb, bdlT, bWt;
  int bwd_chunks = 1;            // token chunks of the router weight gradient (vector path)
  int64_t bwd_tokens_per_chunk = 0;
  bool bwd_mfma = false;         // router products of the backward on the MFMA GEMM
  int bwd_Kp = 0;                // E rounded up to 64
  int64_t bwd_Tp = 0, bwd_T64 = 0;
  int bwd_wsplit = 1;            // K parts of the weight-gradient GEMM
  size_t total = 0;
  // debug canaries: a guard of kCanaryBytes after every region
  int nguards = 0;
  size_t guard_off[kMaxGuards];
  const char* guard_name[kMaxGuards];
};

// Shortest decimal that round-trips the double, as digits D and exponent X:
// cf = D * 10^X.  Returns false for non-finite input.
bool decimal_of(double cf, __int128* D, int* X) {
  if (!isfinite(cf)) return false;
  char buf[64];
  for (int prec = 0; prec <= 17; ++prec) {
    snprintf(buf, sizeof(buf), "%.*e", prec, cf);
    if (strtod(buf, nullptr) == cf) break;
  }
  // buf = "d.ddddde[+-]XX"
  __int128 digits = 0;
  int ndec = 0;
  bool after_point = false;
  const char* p = buf;
  for (; *p && *p != 'e'; ++p) {
    if (*p == '.') { after_point = true; continue; }
    if (*p >= '0' && *p <= '9') {
      digits = digits * 10 + (*p - '0');
      if (after_point) ++ndec;
    }
  }
  int ex = (*p == 'e') ? atoi(p + 1) : 0;
  *D = digits;
  *X = ex - ndec;
  return true;
}

// Capacity C = ceil(T*k*cf/E), exactly, with cf its shortest decimal.
// [Routing guide] "MoE routing, fully explained" (allinfo.ai.kr), "Plain
// explanation" para 5: batch x top-k x capacity factor / experts.
// Every product stays below 2^127: T*k < 2^31, D < 10^18, cf <= 1e6 keeps
// num below 2^31 * 10^24, and den grows only while it is at most num (once
// den > num > 0 the quotient lies in (0, 1) and rounds up to 1).
int64_t exact_capacity(int64_t T, int k, int E, double cf) {
  if (!(cf > 0.0)) return T;  // no limit
  __int128 D;
  int X;
  if (!decimal_of(cf, &D, &X)) return -1;
  __int128 num = static_cast<__int128>(T) * k * D;
  if (num == 0) return 0;
  __int128 den = E;
  for (; X > 0; --X) num *= 10;
  for (; X < 0; ++X) {
    if (den > num) return 1;
    den *= 10;
  }
  __int128 q = (num + den - 1) / den;
  return static_cast<int64_t>(q);
}

int check(const moe_config_t* c) {
  if (!c) return fail(MOE_EINVAL, "cfg is NULL");
  if (c->T < 0) return fail(MOE_EINVAL, "T = %lld must be >= 0", (long long)c->T);
  if (c->d_model <= 0 || c->d_ff <= 0)
    return fail(MOE_EINVAL, "d_model = %d and d_ff = %d must be positive", c->d_model, c->d_ff);
  if (c->n_experts < 1 || c->n_experts > moe::kMaxExperts)
    return fail(MOE_EINVAL, "n_experts = %d must be in [1, %d]", c->n_experts, moe::kMaxExperts);
  if (c->top_k < 1 || c->top_k > c->n_experts)
    return fail(MOE_EINVAL, "top_k = %d must be in [1, n_experts = %d]", c->top_k, c->n_experts);
  if (c->n_shared < 0) return fail(MOE_EINVAL, "n_shared = %d must be >= 0", c->n_shared);
  if (c->gating != MOE_TOPK_THEN_SOFTMAX && c->gating != MOE_SOFTMAX_THEN_TOPK)
    return fail(MOE_EINVAL, "gating = %d is not a moe_gating_t", c->gating);
  if (c->renormalize != 0 && c->renormalize != 1)
    return fail(MOE_EINVAL, "renormalize = %d must be 0 or 1", c->renormalize);
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16)
    return fail(MOE_EINVAL, "dtype = %d is not a moe_dtype_t", c->dtype);
  if (c->ffn_path < MOE_PATH_AUTO || c->ffn_path > MOE_PATH_STREAM)
    return fail(MOE_EINVAL, "ffn_path = %d is not a moe_ffn_path_t", c->ffn_path);
  if (c->overflow < MOE_OVERFLOW_DROP || c->overflow > MOE_OVERFLOW_SEQUENTIAL)
    return fail(MOE_EINVAL, "overflow = %d is not a moe_overflow_t", c->overflow);
  if (c->weight_layout != MOE_WEIGHTS_ROW_MAJOR && c->weight_layout != MOE_WEIGHTS_PACKED)
    return fail(MOE_EINVAL, "weight_layout = %d is not a moe_weight_layout_t", c->weight_layout);
  if (c->out_fp32 != 0 && c->out_fp32 != 1)
    return fail(MOE_EINVAL, "out_fp32 = %d must be 0 or 1", c->out_fp32);
  if (isnan(c->capacity_factor) || c->capacity_factor > 1e6)
    return fail(MOE_EINVAL, "capacity_factor must be a number <= 1e6");
  if (c->T * static_cast<int64_t>(c->top_k) >= (int64_t(1) << 31))
    return fail(MOE_EINVAL, "T * top_k must be < 2^31");
  if (static_cast<int64_t>(c->n_experts + c->n_shared) * c->d_model * c->d_ff >= (int64_t(1) << 40))
    return fail(MOE_EINVAL, "expert weights too large");
  if (c->dtype == MOE_DTYPE_BF16) {
    if (c->d_model % 64 != 0 || c->d_ff % 64 != 0)
      return fail(MOE_EUNSUPPORTED, "bf16 layers need d_model and d_ff divisible by 64 (got %d, %d)",
                  c->d_model, c->d_ff);
  } else {
    if (c->ffn_path == MOE_PATH_STREAM)
      return fail(MOE_EUNSUPPORTED, "fp32 layers run on the fp32 grouped kernels only");
    if (c->weight_layout == MOE_WEIGHTS_PACKED)
      return fail(MOE_EUNSUPPORTED, "packed weights are for bf16 layers");
  }
  return MOE_OK;
}

// Packed weights: block widths of W1/W3 and of W2, and the padded widths.
constexpr int kPackW13 = 128;
constexpr int kPackW2 = 256;
int64_t pad_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// K parts for a GEMM with `tiles` output tiles and `ksteps` 64-deep K
// steps: enough for ~512 workgroups (more than 1 only when the tiles alone
// give fewer than 256).  The kernels split K into near-equal runs of steps,
// so the count need not divide ksteps.
int split_for(int64_t tiles, int ksteps, bool force) {
  if (tiles <= 0) return 1;
  if (!force && tiles >= 256) return 1;
  int64_t ks = (512 + tiles - 1) / tiles;
  if (ks > ksteps) ks = ksteps;
  if (ks > 64) ks = 64;
  if (ks < 1) ks = 1;
  return static_cast<int>(ks);
}

void add(Region& r, size_t bytes, size_t& cursor) {
  r.off = cursor;
  r.bytes = bytes;
  cursor = align_up(cursor + bytes);
}
// add() plus, with canaries on, a guard after the region.
void add_guarded(Plan* p, Region& r, size_t bytes, size_t& cursor, const char* name) {
  add(r, bytes, cursor);
  if (g_canaries.load(std::memory_order_relaxed) && p->nguards < kMaxGuards) {
    p->guard_off[p->nguards] = cursor;
    p->guard_name[p->nguards] = name;
    ++p->nguards;
    cursor = align_up(cursor + kCanaryBytes);
  }
}

int make_plan(const moe_config_t* c, Plan* p) {
  int rc = check(c);
  if (rc != MOE_OK) return rc;
  p->T = c->T;
  p->d = c->d_model;
  p->F = c->d_ff;
  p->E = c->n_experts;
  p->k = c->top_k;
  p->S = c->n_shared;
  p->gating = c->gating;
  p->renorm = c->renormalize;
  p->bf16 = c->dtype == MOE_DTYPE_BF16;
  p->path = c->ffn_path;
  p->capacity = exact_capacity(c->T, c->top_k, c->n_experts, c->capacity_factor);
  if (p->capacity < 0) return fail(MOE_EINVAL, "capacity_factor is not finite");
  p->overflow = c->overflow;
  p->Ceff = static_cast<int>(p->capacity < p->T ? p->capacity : p->T);
  // Sequential rounds keep every assignment: one launch runs all the rounds'
  // rows, so the dispatch sees no limit (the rounds are reported).
  if (p->overflow == MOE_OVERFLOW_SEQUENTIAL) p->Ceff = static_cast<int>(p->T);
  p->TK = p->T * p->k;
  p->rows_max = p->TK;
  if (static_cast<int64_t>(p->E) * p->Ceff < p->rows_max) p->rows_max = static_cast<int64_t>(p->E) * p->Ceff;
  p->nblk_dispatch = static_cast<int>((p->TK + moe::kDispatchChunk - 1) / moe::kDispatchChunk);
  const int G = moe::topk_group_size(p->E);
  const int groups = 256 / G;
  int64_t tpb = (p->T + 1023) / 1024;
  tpb = (tpb + groups - 1) / groups * groups;
  if (tpb < groups) tpb = groups;
  p->topk_tpb = static_cast<int>(tpb);
  p->topk_blocks = static_cast<int>((p->T + tpb - 1) / tpb);
  // Short batches: top-k, gates and dispatch run as one kernel in one
  // workgroup (its softmax statistics come as a single partial row).
  p->small_route = p->T > 0 && p->T <= moe::kSmallT && p->TK <= moe::kSmallTK &&
                   p->overflow != MOE_OVERFLOW_REROUTE;
  if (p->small_route) {
    p->topk_blocks = 1;
    p->topk_tpb = static_cast<int>(p->T);
  }
  // M-tile of the routed GEMMs, from the average rows per hit expert (the
  // tile list is built for it; the M-tile picks the kernel shape):
  //   <= 48        32 rows (short batches: the weights stream once);
  //   384 .. 1536 128 rows, two workgroups per CU (barriers and tile set-up
  //               of one overlap the other's MFMAs), token rows gathered into
  //               a K-blocked copy first;
  //   otherwise   256 rows, one workgroup per CU: with a few hundred rows (as
  //               with many fine-grained experts) one M-tile per expert reads
  //               each weight tile once; with thousands, each weight tile is
  //               fetched for half as many M-tiles.
  if (p->bf16) {
    const int64_t hit = p->TK < p->E ? p->TK : p->E;
    if (hit > 0 && p->TK <= 48 * hit) p->bm = moe::kGroupedBMShort;
    else if (hit > 0 && p->TK >= 384 * hit && p->TK <= 1536 * hit) p->bm = moe::kGroupedBM;
    else p->bm = moe::kGroupedBMWide;
    p->static_bm = p->T <= 64 ? moe::kGroupedBMShort : moe::kGroupedBM;
  } else {
    p->bm = p->static_bm = moe::kF32BM;
  }
  p->max_mtiles = static_cast<int>(p->rows_max / p->bm + p->E);
  // Long batches: GEMM1 writes H K-blocked, so each K step of a GEMM2 tile
  // reads one contiguous run of memory instead of 64-byte pieces of rows.
  // With 128-row tiles, the kept token rows are likewise first gathered into
  // a slot-ordered K-blocked copy for GEMM1.  Short batches read the few rows
  // directly.
  p->blocked = p->bf16 && p->bm != moe::kGroupedBMShort;
  p->gather_x = p->blocked && p->bm == moe::kGroupedBM;
  // Router scores x W_gate on the MFMA GEMM when the weight rows are 16-byte
  // aligned; K is split so that short batches give more workgroups, and the
  // top-k pass adds the parts in a fixed order.  At most 16 parts: the top-k
  // pass reads every part of a score before it can rank, 8 loads in flight
  // at a time, so each 8 parts cost it a memory round trip.
  p->mfma_router = p->bf16 && (p->E % 8 == 0);
  if (p->mfma_router) {
    const int kk = p->d / 64;
    const int64_t mt = (p->T + p->static_bm - 1) / p->static_bm;
    int64_t ks = mt > 0 ? (512 + mt - 1) / mt : 1;
    if (ks > 16) ks = 16;
    // Many experts (E > 64): each part adds 4 T E bytes of partial sums to
    // write and read back, and at most 8 parts measured faster (160 experts:
    // router + top-k 45 against 51 us with 16).
    if (p->E > 64 && ks > 8) ks = 8;
    if (ks > kk) ks = kk;
    if (ks < 1) ks = 1;
    while (kk % ks) --ks;
    p->router_split = static_cast<int>(ks);
    // Short batches with 8 or 16 experts: one wavefront per K part, at most
    // 8 parts (one load round in the top-k pass).
    if (moe::router_parts_fit(p->T, p->E, p->d)) {
      int np = kk < 8 ? kk : 8;
      while (kk % np) --np;
      p->router_split = np;
      p->parts_router = true;
    } else {
      // Up to 64 experts: a kernel whose weight operand is E columns wide
      // rather than a 256-wide GEMM tile, in parts of 256 columns where d
      // allows at most 16 of them (each wavefront then has its part's token
      // loads in flight at once), else in the parts above.
      const int np = p->d % 256 == 0 ? p->d / 256 : 0;
      if (np >= 1 && np <= 16 && moe::router_narrow_fit(p->T, p->E, p->d, np)) {
        p->router_split = np;
        p->narrow_router = true;
      } else if (moe::router_narrow_fit(p->T, p->E, p->d, p->router_split)) {
        p->narrow_router = true;
      }
    }
  }
  // Down projections with few tiles (short batches: a few rows per expert)
  // split K so ~512 workgroups stream the weights; the combine adds the
  // parts in a fixed order.  The estimate of routed M-tiles assumes at most
  // min(E, T*k) experts are hit.  The grouped path never splits; the
  // streaming path always splits as far as the workgroup target allows.
  // Short batches' down projection takes 128-wide weight tiles (two
  // workgroups per CU), so the same workgroup count needs half the K parts.
  if (p->bf16 && p->path != MOE_PATH_GROUPED) {
    const int ntn2 = p->bm == moe::kGroupedBMShort ? (p->d + 127) / 128 : (p->d + 255) / 256;
    const int64_t hit = p->TK < p->E ? p->TK : p->E;
    const int64_t mt_est = p->rows_max / p->bm + hit;
    p->ffn2_split = split_for(mt_est * ntn2, p->F / 64, p->path == MOE_PATH_STREAM);
    // Long batches whose down-projection tiles fill one whole round of
    // resident workgroups and then a last round less than half full (e.g.
    // 592 tiles on 512 slots): two K parts turn that into fuller rounds.
    if (p->path == MOE_PATH_AUTO && p->ffn2_split == 1 && p->bm != moe::kGroupedBMShort) {
      const int64_t slots = static_cast<int64_t>(device_cus()) * (p->bm == moe::kGroupedBM ? 2 : 1);
      const int64_t t = mt_est * ntn2;
      if (slots > 0 && t > slots && t < 4 * slots && (t % slots) != 0 && (t % slots) <= slots / 2) {
        p->ffn2_split = 2;
        // where to cut K is decided on the device from the tiles that exist
        p->ffn2_kcut_slots = static_cast<int>(slots);
      }
    }
    if (p->S > 0) {
      const int64_t mts = (p->T + p->static_bm - 1) / p->static_bm;
      const int ntn2s = (p->d + 255) / 256;   // the shared experts keep 256-wide tiles
      p->shared2_split = split_for(mts * ntn2s, p->S * p->F / 64, p->path == MOE_PATH_STREAM);
    }
  }

  const size_t es = p->bf16 ? 2 : 4;
  size_t cur = 0;
  add_guarded(p, p->logits, sizeof(float) * p->T * p->E, cur, "logits");
  add_guarded(p, p->lpart, sizeof(float) * (p->mfma_router ? p->router_split : 0) * p->T * p->E, cur, "lpart");
  add_guarded(p, p->idx, sizeof(int32_t) * p->TK, cur, "idx");
  add_guarded(p, p->w, sizeof(float) * p->TK, cur, "w");
  add_guarded(p, p->lrank, sizeof(int32_t) * p->TK, cur, "lrank");
  add_guarded(p, p->blkcnt, sizeof(int32_t) * static_cast<size_t>(p->nblk_dispatch) * p->E, cur, "blkcnt");
  add_guarded(p, p->counts, sizeof(int32_t) * p->E, cur, "counts");
  add_guarded(p, p->kcount, sizeof(int32_t) * p->E, cur, "kcount");
  add_guarded(p, p->offsets, sizeof(int32_t) * (p->E + 1), cur, "offsets");
  add_guarded(p, p->slot, sizeof(int32_t) * p->TK, cur, "slot");
  add_guarded(p, p->perm, sizeof(int32_t) * p->TK, cur, "perm");
  add_guarded(p, p->tiles, sizeof(moe::Tile) * (p->max_mtiles + 1), cur, "tiles");
  add_guarded(p, p->ntiles, sizeof(int32_t) * 4, cur, "ntiles");
  add_guarded(p, p->tstart, sizeof(int32_t) * (p->E + 1), cur, "tstart");
  add_guarded(p, p->ppart, sizeof(float) * static_cast<size_t>(p->topk_blocks) * p->E, cur, "ppart");
  add_guarded(p, p->hpart, sizeof(float) * p->topk_blocks, cur, "hpart");
  add_guarded(p, p->stats, sizeof(double) * 8, cur, "stats");
  add_guarded(p, p->H, es * p->rows_max * p->F, cur, "H");
  add_guarded(p, p->Hs, es * p->T * p->S * p->F, cur, "Hs");
  // The routed down projection's rows stay fp32 (K parts summed by the
  // combine), so the only roundings before the output's are the hidden rows'.
  add_guarded(p, p->Y, sizeof(float) * p->ffn2_split * p->rows_max * p->d, cur, "Y");
  add_guarded(p, p->Ys, sizeof(float) * p->shared2_split * (p->S > 0 ? p->T : 0) * p->d, cur, "Ys");
  add_guarded(p, p->Xb, p->gather_x ? es * p->rows_max * p->d : 0, cur, "Xb");
  const size_t rr = p->overflow == MOE_OVERFLOW_REROUTE ? sizeof(int32_t) * p->TK : 0;
  add_guarded(p, p->ovf, rr, cur, "ovf");
  add_guarded(p, p->xdest, rr, cur, "xdest");
  add_guarded(p, p->xrel, rr, cur, "xrel");
  // Router backward.  bf16 layers: both router products run on the MFMA
  // GEMM with bf16 score gradients; the weight gradient's K (tokens) is
  // split for ~512 workgroups with at most 16 MiB of partial sums.  fp32
  // layers: the weight gradient sums x^T dlogits on vector kernels over
  // token chunks of at least 256 tokens, with at most 16 MiB of partials.
  p->bwd_mfma = p->bf16;
  if (p->bwd_mfma) {
    p->bwd_Kp = (p->E + 63) / 64 * 64;
    p->bwd_Tp = (p->T + 63) / 64 * 64;
    p->bwd_T64 = p->T / 64 * 64;
    const int64_t ed = static_cast<int64_t>(p->E) * p->d;
    const int bmw = p->E <= 64 ? moe::kGroupedBMShort : moe::kGroupedBM;
    const int bk = bmw == moe::kGroupedBMShort ? 64 : 32;
    const int64_t tiles = ((p->E + bmw - 1) / bmw) * ((p->d + 255) / 256);
    int64_t ks = (512 + tiles - 1) / tiles;
    const int64_t nk = p->bwd_T64 / bk;
    if (ks > nk) ks = nk;
    const int64_t cap = (int64_t(16) << 20) / (4 * ed);
    if (ks > cap) ks = cap;
    if (ks > 64) ks = 64;
    if (ks < 1) ks = 1;
    p->bwd_wsplit = static_cast<int>(ks);
    add_guarded(p, p->gpart, sizeof(float) * (ks * ed + ed + p->E), cur, "gpart");
    add_guarded(p, p->bdlb, 2 * static_cast<size_t>(p->T) * p->bwd_Kp, cur, "bdlb");
    add_guarded(p, p->bdlT, 2 * static_cast<size_t>(p->E) * p->bwd_Tp, cur, "bdlT");
    add_guarded(p, p->bWt, 2 * static_cast<size_t>(p->bwd_Kp) * p->d, cur, "bWt");
  } else {
    const int64_t per = static_cast<int64_t>(p->d) * p->E + p->E;
    int64_t nc = (p->T + 255) / 256;
    const int64_t cap = (int64_t(16) << 20) / (4 * per);
    if (nc > cap) nc = cap;
    if (nc > 64) nc = 64;
    if (nc < 1) nc = 1;
    p->bwd_tokens_per_chunk = (p->T + nc - 1) / nc;
    if (p->bwd_tokens_per_chunk < 1) p->bwd_tokens_per_chunk = 1;
    p->bwd_chunks = static_cast<int>((p->T + p->bwd_tokens_per_chunk - 1) / p->bwd_tokens_per_chunk);
    if (p->bwd_chunks < 1) p->bwd_chunks = 1;
    add_guarded(p, p->gpart, sizeof(float) * per * p->bwd_chunks, cur, "gpart");
  }
  p->total = cur;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, const Region& r) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + r.off);
}

// The kernels read and write x, W_gate, the expert weights and out with
// 16-byte vector loads and global -> LDS transfers, so those pointers must be
// 16-byte aligned (device allocations are; a view that starts part-way into
// an allocation need not be).  NULL passes here; it is checked on its own.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return false;
  return true;
}

int check_workspace(const moe_config_t* c, const Plan& p) {
  if (p.T == 0) return MOE_OK;
  if (!c->workspace) return fail(MOE_EWORKSPACE, "workspace is NULL (need %zu bytes)", p.total);
  if (reinterpret_cast<uintptr_t>(c->workspace) % kAlign != 0)
    return fail(MOE_EWORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (c->workspace_bytes < p.total)
    return fail(MOE_EWORKSPACE, "workspace has %zu bytes, need %zu", c->workspace_bytes, p.total);
  return MOE_OK;
}

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return fail(MOE_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

// Debug canaries: write every guard of the plan (see kCanaryBytes).
int arm_canaries(const Plan& p, void* ws, hipStream_t s) {
  for (int i = 0; i < p.nguards; ++i)
    HIP_TRY(hipMemsetAsync(static_cast<char*>(ws) + p.guard_off[i], kCanaryByte, kCanaryBytes, s));
  return MOE_OK;
}

// Step 1: router scores.  Returns, through lsrc/nsplit/bias, where the
// top-k pass finds them: K-split partial sums of the MFMA GEMM (bias added
// by the top-k pass) or complete scores from the vector kernels.
struct Scores {
  const float* lsrc;
  int nsplit;
  int64_t split_stride;
  const float* bias;
};

int run_router(const Plan& p, void* ws, const void* x, const void* W_gate,
               const float* bias, hipStream_t s, Scores* sc) {
  if (p.parts_router) {
    Timed t("router", s);
    HIP_TRY(moe::launch_router_parts(x, W_gate, static_cast<int>(p.T), p.d, p.E, p.router_split,
                                     at<float>(ws, p.lpart), s));
    *sc = Scores{at<float>(ws, p.lpart), p.router_split, p.T * p.E, bias};
  } else if (p.narrow_router) {
    Timed t("router", s);
    HIP_TRY(moe::launch_router_narrow(x, W_gate, p.T, p.d, p.E, p.router_split,
                                      at<float>(ws, p.lpart), s));
    *sc = Scores{at<float>(ws, p.lpart), p.router_split, p.T * p.E, bias};
  } else if (p.mfma_router) {
    moe::GroupedGemm r{};
    r.A = x; r.lda = p.d; r.perm = nullptr; r.topk = 1;
    r.B = W_gate; r.B3 = nullptr; r.b_stride = 0; r.group_base = 0; r.ldb = p.E;
    r.K = p.d; r.N = p.E; r.ngroups_n = 1; r.C = at<float>(ws, p.lpart); r.ldc = p.E;
    r.c_group_col = 0; r.tiles = nullptr; r.ntiles = nullptr; r.tstart = nullptr;
    r.n_experts = 1; r.static_rows = static_cast<int>(p.T);
    r.max_mtiles = static_cast<int>((p.T + p.static_bm - 1) / p.static_bm);
    r.bm = p.static_bm;
    r.ksplit = p.router_split; r.c_split = p.T * p.E;
    Timed t("router", s);
    HIP_TRY(moe::launch_grouped_plain_bf16(r, s));
    *sc = Scores{at<float>(ws, p.lpart), p.router_split, p.T * p.E, bias};
  } else {
    Timed t("router", s);
    HIP_TRY(moe::launch_router(x, W_gate, bias, at<float>(ws, p.logits), p.T, p.d, p.E,
                               p.bf16, s));
    *sc = Scores{at<float>(ws, p.logits), 1, 0, nullptr};
  }
  return MOE_OK;
}

// Steps 2-3 (top-k, gates, dispatch) from router scores `sc`; the summed
// scores are also written to logits_out when it is given.  Rerouting reads
// the full scores again: complete ones in place, partial sums as the top-k
// pass stores them (in logits_out, else in the workspace).
int run_route(const Plan& p, void* ws, const Scores& sc, float* logits_out, int32_t* idx,
              float* w, hipStream_t s) {
  moe::Reroute rr{};
  const moe::Reroute* rrp = nullptr;
  if (p.overflow == MOE_OVERFLOW_REROUTE) {
    if (sc.nsplit == 1 && sc.bias == nullptr) {
      rr.logits = sc.lsrc;
    } else {
      if (!logits_out) logits_out = at<float>(ws, p.logits);
      rr.logits = logits_out;
    }
    rr.k = p.k;
    rr.ovf = at<int32_t>(ws, p.ovf);
    rr.xdest = at<int32_t>(ws, p.xdest);
    rr.xrel = at<int32_t>(ws, p.xrel);
    rrp = &rr;
  }
  if (p.small_route) {
    Timed t("route_small", s);
    HIP_TRY(moe::launch_route_small(
        sc.lsrc, sc.nsplit, sc.split_stride, sc.bias, logits_out, static_cast<int>(p.T), p.E,
        p.k, p.gating, p.renorm, idx, w, at<float>(ws, p.ppart), at<float>(ws, p.hpart),
        p.Ceff, at<int32_t>(ws, p.counts), at<int32_t>(ws, p.kcount), at<int32_t>(ws, p.offsets),
        at<int32_t>(ws, p.slot), at<int32_t>(ws, p.perm), p.bm, at<moe::Tile>(ws, p.tiles),
        at<int32_t>(ws, p.ntiles), at<int32_t>(ws, p.tstart), s));
    return MOE_OK;
  }
  {
    Timed t("topk_gate", s);
    HIP_TRY(moe::launch_topk_gate(sc.lsrc, sc.nsplit, sc.split_stride, sc.bias, logits_out,
                                  p.T, p.E, p.k, p.gating, p.renorm, idx, w,
                                  at<float>(ws, p.ppart), at<float>(ws, p.hpart),
                                  p.topk_blocks, p.topk_tpb, s));
  }
  {
    Timed t("dispatch", s);
    HIP_TRY(moe::launch_dispatch(idx, p.TK, p.E, p.Ceff, at<int32_t>(ws, p.lrank),
                                 at<int32_t>(ws, p.blkcnt), at<int32_t>(ws, p.counts),
                                 at<int32_t>(ws, p.kcount), at<int32_t>(ws, p.offsets),
                                 at<int32_t>(ws, p.slot), at<int32_t>(ws, p.perm), p.bm,
                                 at<moe::Tile>(ws, p.tiles), at<int32_t>(ws, p.ntiles),
                                 at<int32_t>(ws, p.tstart), rrp, s));
  }
  return MOE_OK;
}

int fill_stats(const Plan& p, void* ws, hipStream_t s, moe_stats_t* st,
               const int32_t* counts_dev, const int32_t* kcount_dev) {
  memset(&st->aux_loss, 0, sizeof(double) * 5);
  st->capacity = p.capacity;
  st->assignments = p.TK;
  st->dropped = 0;
  st->overflowed = 0;
  st->rerouted = 0;
  st->rounds = 0;
  if (p.T == 0) {
    if (st->counts) memset(st->counts, 0, sizeof(int64_t) * p.E);
    if (st->kept) memset(st->kept, 0, sizeof(int64_t) * p.E);
    return MOE_OK;
  }
  {
    Timed t("stats", s);
    HIP_TRY(moe::launch_stats(at<float>(ws, p.ppart), at<float>(ws, p.hpart), p.topk_blocks,
                              counts_dev, kcount_dev, p.T, p.k, p.E, at<double>(ws, p.stats), s));
  }
  double out[8];
  int32_t cnt[moe::kMaxExperts] = {}, kc[moe::kMaxExperts] = {};
  HIP_TRY(hipMemcpyAsync(out, at<double>(ws, p.stats), sizeof(double) * 6, hipMemcpyDeviceToHost, s));
  if (counts_dev)
    HIP_TRY(hipMemcpyAsync(cnt, counts_dev, sizeof(int32_t) * p.E, hipMemcpyDeviceToHost, s));
  if (kcount_dev)
    HIP_TRY(hipMemcpyAsync(kc, kcount_dev, sizeof(int32_t) * p.E, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  st->aux_loss = out[0];
  st->aux_loss_kept = out[1];
  st->overflow_rate = out[2];
  st->entropy_load = out[3];
  st->entropy_token = out[4];
  st->dropped = static_cast<int64_t>(out[5]);
  for (int e = 0; e < p.E; ++e) {
    if (st->counts) st->counts[e] = cnt[e];
    if (st->kept) st->kept[e] = kc[e];
  }
  // Assignments beyond their chosen expert's C slots, and the C-row rounds
  // the busiest chosen expert needs; what is not dropped of the overflow
  // went to spare experts or to later rounds.
  for (int e = 0; e < p.E; ++e) {
    if (cnt[e] > p.capacity) st->overflowed += cnt[e] - p.capacity;
    if (cnt[e] > 0 && p.capacity > 0) {
      const int64_t r = (cnt[e] + p.capacity - 1) / p.capacity;
      if (r > st->rounds) st->rounds = r;
    }
  }
  if (p.overflow == MOE_OVERFLOW_REROUTE) st->rerouted = st->overflowed - st->dropped;
  return MOE_OK;
}

// ------------------------------------------------------- allocation-free
// Scratch of moe_forward_noalloc, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): one fixed array in device memory, which every GPU the library
// runs on holds until the process ends.  In host code `scratch` names a host
// stand-in, not the device array: kernels and copies only ever get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr after a failure
// (moe_last_error says why).
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(MOE_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(MOE_EHIP, "device %d is beyond the %d devices the scratch table covers", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || p == nullptr) {
      fail(MOE_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
           hipGetErrorString(r));
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

int moe_check_config(const moe_config_t* cfg) {
  int rc = check(cfg);
  if (rc == MOE_OK) g_err.clear();
  return rc;
}

size_t moe_workspace_size(const moe_config_t* cfg) {
  Plan p;
  if (make_plan(cfg, &p) != MOE_OK) return 0;
  return p.total;
}

int64_t moe_capacity(const moe_config_t* cfg) {
  Plan p;
  if (make_plan(cfg, &p) != MOE_OK) return -1;
  return p.capacity;
}

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_forward(const void* x, const void* W_gate, const void* W1, const void* W3,
                const void* W2, const moe_config_t* cfg, void* out, moe_stats_t* stats) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (p.T > 0 && (!x || !W_gate || !W1 || !W3 || !W2 || !out))
    return fail(MOE_EINVAL, "x, W_gate, W1, W3, W2 and out must be non-NULL");
  if (p.T > 0 && !aligned16({x, W_gate, W1, W3, W2, out}))
    return fail(MOE_EINVAL, "x, W_gate, W1, W3, W2 and out must be 16-byte aligned");
  rc = check_workspace(cfg, p);
  if (rc != MOE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  if (p.T == 0) {
    if (stats) fill_stats(p, nullptr, s, stats, nullptr, nullptr);
    g_err.clear();
    return MOE_OK;
  }
  void* ws = cfg->workspace;
  rc = arm_canaries(p, ws, s);
  if (rc != MOE_OK) return rc;
  int32_t* idx = at<int32_t>(ws, p.idx);
  float* w = at<float>(ws, p.w);
  Scores sc;
  rc = run_router(p, ws, x, W_gate, cfg->logit_bias, s, &sc);
  if (rc != MOE_OK) return rc;
  // the summed scores stay in the workspace for the router backward
  rc = run_route(p, ws, sc, sc.lsrc == at<float>(ws, p.logits) ? nullptr : at<float>(ws, p.logits),
                 idx, w, s);
  if (rc != MOE_OK) return rc;

  // GEMM1 (routed): H[slot] = silu(x[token] W1[e]) * (x[token] W3[e])
  // Packed weights: W1/W3 rows padded to F13 columns, W2 rows to D2.
  const bool packed = cfg->weight_layout == MOE_WEIGHTS_PACKED;
  const int F13 = packed ? static_cast<int>(pad_to(p.F, kPackW13)) : p.F;
  const int D2 = packed ? static_cast<int>(pad_to(p.d, kPackW2)) : p.d;
  moe::GroupedGemm g1{};
  g1.A = x; g1.lda = p.d; g1.perm = at<int32_t>(ws, p.perm); g1.topk = p.k;
  g1.B = W1; g1.B3 = W3; g1.b_stride = static_cast<int64_t>(p.d) * F13; g1.group_base = 0;
  g1.ldb = F13; g1.b_block_cols = packed ? kPackW13 : 0;
  g1.K = p.d; g1.N = p.F; g1.ngroups_n = 1; g1.C = at<void>(ws, p.H); g1.ldc = p.F;
  g1.c_group_col = 0; g1.tiles = at<moe::Tile>(ws, p.tiles); g1.ntiles = at<int32_t>(ws, p.ntiles);
  g1.tstart = at<int32_t>(ws, p.tstart); g1.n_experts = p.E; g1.ksplit = 1; g1.c_split = 0;
  g1.static_rows = 0; g1.max_mtiles = p.max_mtiles; g1.bm = p.bm;
  // Short batches hitting several experts: the SwiGLU GEMM takes 128-wide B
  // tiles (two workgroups per CU), so more CUs stream the weights at once.
  g1.narrow_n = p.bm == moe::kGroupedBMShort && (p.TK < p.E ? p.TK : p.E) >= 4;
  if (p.gather_x) {
    Timed t("gather", s);
    HIP_TRY(moe::launch_gather_blocked(x, p.d, at<int32_t>(ws, p.perm), p.k,
                                       at<int32_t>(ws, p.offsets) + p.E, p.rows_max, p.d,
                                       at<void>(ws, p.Xb), s));
    g1.A = at<void>(ws, p.Xb); g1.perm = nullptr; g1.a_block_rows = p.rows_max;
  }
  if (p.blocked) g1.c_block_rows = p.rows_max;
  // GEMM2 (routed): Y[slot] = H[slot] W2[e]
  moe::GroupedGemm g2 = g1;
  g2.A = at<void>(ws, p.H); g2.lda = p.F; g2.perm = nullptr; g2.B = W2; g2.B3 = nullptr;
  g2.ldb = D2; g2.b_stride = static_cast<int64_t>(p.F) * D2; g2.b_block_cols = packed ? kPackW2 : 0;
  g2.K = p.F; g2.N = p.d; g2.C = at<void>(ws, p.Y); g2.ldc = p.d;
  g2.ksplit = p.ffn2_split; g2.c_split = p.rows_max * p.d; g2.kcut_slots = p.ffn2_kcut_slots;
  g2.narrow_n = p.bm == moe::kGroupedBMShort ? 1 : 0;
  g2.a_block_rows = g1.c_block_rows;   // GEMM2 reads H as GEMM1 wrote it
  g2.c_block_rows = 0;
  // Shared experts: all T token rows; GEMM1 lays the S experts side by side
  // along N into Hs [T, S*F]; GEMM2 contracts the S*F hidden columns against
  // the S stacked W2 blocks in one pass (their sum).
  moe::GroupedGemm s1{}, s2{};
  if (p.S > 0) {
    s1 = g1;
    s1.A = x; s1.a_block_rows = 0; s1.c_block_rows = p.blocked ? p.T : 0; s1.narrow_n = 0;
    s1.perm = nullptr; s1.group_base = p.E; s1.ngroups_n = p.S; s1.C = at<void>(ws, p.Hs);
    s1.ldc = static_cast<int64_t>(p.S) * p.F; s1.c_group_col = p.F; s1.tiles = nullptr;
    s1.ntiles = nullptr; s1.tstart = nullptr; s1.static_rows = static_cast<int>(p.T);
    s1.max_mtiles = static_cast<int>((p.T + p.static_bm - 1) / p.static_bm);
    s1.bm = p.static_bm;
    s2 = s1;
    s2.a_block_rows = s1.c_block_rows; s2.c_block_rows = 0;
    s2.A = at<void>(ws, p.Hs); s2.lda = static_cast<int64_t>(p.S) * p.F; s2.B = W2; s2.B3 = nullptr;
    s2.b_stride = static_cast<int64_t>(p.F) * D2; s2.group_base = p.E; s2.ngroups_n = 1;
    s2.ldb = D2; s2.b_block_cols = packed ? kPackW2 : 0;
    s2.K = p.S * p.F; s2.N = p.d; s2.C = at<void>(ws, p.Ys); s2.ldc = p.d; s2.c_group_col = 0;
    s2.ksplit = p.shared2_split; s2.c_split = p.T * p.d;
  }
  if (p.bf16) {
    {
      Timed t("ffn1_swiglu", s);
      HIP_TRY(moe::launch_grouped_swiglu_bf16(g1, s));
    }
    if (p.S > 0) {
      Timed t("ffn1_swiglu_shared", s);
      HIP_TRY(moe::launch_grouped_swiglu_bf16(s1, s));
    }
    {
      Timed t("ffn2", s);
      HIP_TRY(moe::launch_grouped_plain_bf16(g2, s));
    }
    if (p.S > 0) {
      Timed t("ffn2_shared", s);
      HIP_TRY(moe::launch_grouped_plain_bf16(s2, s));
    }
  } else {
    {
      Timed t("ffn1_swiglu_f32", s);
      HIP_TRY(moe::launch_grouped_swiglu_f32(g1, s));
    }
    if (p.S > 0) {
      Timed t("ffn1_swiglu_f32_shared", s);
      HIP_TRY(moe::launch_grouped_swiglu_f32(s1, s));
    }
    {
      Timed t("ffn2_f32", s);
      HIP_TRY(moe::launch_grouped_plain_f32(g2, s));
    }
    if (p.S > 0) {
      Timed t("ffn2_f32_shared", s);
      HIP_TRY(moe::launch_grouped_plain_f32(s2, s));
    }
  }
  {
    Timed t("combine", s);
    HIP_TRY(moe::launch_combine(at<float>(ws, p.Y), p.ffn2_split, p.rows_max * p.d,
                                at<int32_t>(ws, p.slot), w,
                                p.S > 0 ? at<float>(ws, p.Ys) : nullptr, p.shared2_split,
                                p.T * p.d, p.T, p.k, p.d, out, p.bf16 && !cfg->out_fp32, s));
  }
  if (stats) {
    rc = fill_stats(p, ws, s, stats, at<int32_t>(ws, p.counts), at<int32_t>(ws, p.kcount));
    if (rc != MOE_OK) return rc;
  }
  g_err.clear();
  return MOE_OK;
}

int moe_forward_noalloc(const void* x, const void* W_gate, const void* W1, const void* W3,
                        const void* W2, const moe_config_t* cfg, void* out, moe_stats_t* stats) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (p.total > kNoAllocScratchBytes)
    return fail(MOE_EWORKSPACE,
                "this layer needs %zu bytes of scratch; moe_forward_noalloc holds %zu "
                "(use moe_forward with a workspace)", p.total, kNoAllocScratchBytes);
  moe_config_t c = *cfg;
  c.workspace = nullptr;
  c.workspace_bytes = 0;
  if (p.T > 0) {
    if (!x || !W_gate || !W1 || !W3 || !W2 || !out)
      return fail(MOE_EINVAL, "x, W_gate, W1, W3, W2 and out must be non-NULL");
    void* ws = scratch_on_current_device();
    if (!ws) return MOE_EHIP;
    c.workspace = ws;
    c.workspace_bytes = kNoAllocScratchBytes;
  }
  return moe_forward(x, W_gate, W1, W3, W2, &c, out, stats);
}

int moe_router_backward(const void* x, const void* W_gate, const void* dout, double aux_coef,
                        double entropy_coef, const moe_config_t* cfg, float* dlogits,
                        float* dW_gate, float* dbias, float* dx) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (!isfinite(aux_coef) || !isfinite(entropy_coef))
    return fail(MOE_EINVAL, "aux_coef and entropy_coef must be finite");
  if (p.T == 0) {
    g_err.clear();
    return MOE_OK;
  }
  if (!dout || !dlogits) return fail(MOE_EINVAL, "dout and dlogits must be non-NULL");
  if (dW_gate && !x) return fail(MOE_EINVAL, "x must be non-NULL when dW_gate is requested");
  if (dx && !W_gate) return fail(MOE_EINVAL, "W_gate must be non-NULL when dx is requested");
  if (!aligned16({x, W_gate})) return fail(MOE_EINVAL, "x and W_gate must be 16-byte aligned");
  rc = check_workspace(cfg, p);
  if (rc != MOE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  void* ws = cfg->workspace;
  rc = arm_canaries(p, ws, s);
  if (rc != MOE_OK) return rc;
  moe::RouterBackward b{};
  b.x = x; b.Wg = W_gate; b.dout = dout;
  b.Y = at<void>(ws, p.Y); b.ysplit = p.ffn2_split;
  b.ystride = p.rows_max * p.d;
  b.rows = p.rows_max;
  b.vec4 = p.d % 4 == 0 && reinterpret_cast<uintptr_t>(dout) % (4 * (p.bf16 ? 2 : 4)) == 0;
  b.slot = at<int32_t>(ws, p.slot); b.idx = at<int32_t>(ws, p.idx); b.w = at<float>(ws, p.w);
  b.logits = at<float>(ws, p.logits); b.counts = at<int32_t>(ws, p.counts);
  b.T = p.T; b.k = p.k; b.E = p.E; b.d = p.d; b.bf16 = p.bf16;
  b.chosen_softmax = (p.gating == MOE_TOPK_THEN_SOFTMAX || p.renorm) ? 1 : 0;
  b.aux_scale = static_cast<float>(aux_coef * p.E / static_cast<double>(p.T));
  b.ent_scale = static_cast<float>(entropy_coef / static_cast<double>(p.T));
  b.inv_tk = static_cast<float>(1.0 / (static_cast<double>(p.T) * p.k));
  b.dlogits = dlogits; b.dW = dW_gate; b.dbias = dbias; b.dx = dx;
  b.part = at<float>(ws, p.gpart);
  b.bpart = b.part + static_cast<int64_t>(p.bwd_chunks) * p.d * p.E;
  b.nchunk = p.bwd_chunks; b.tokens_per_chunk = p.bwd_tokens_per_chunk;
  b.mfma = p.bwd_mfma; b.Kp = p.bwd_Kp; b.Tp = p.bwd_Tp; b.T64 = p.bwd_T64;
  b.wsplit = p.bwd_wsplit;
  b.dlb = at<uint16_t>(ws, p.bdlb); b.dlT = at<uint16_t>(ws, p.bdlT); b.Wt = at<uint16_t>(ws, p.bWt);
  {
    Timed t("gate_backward", s);
    HIP_TRY(moe::launch_gate_backward(b, s));
  }
  if (p.bwd_mfma && (dW_gate || dx)) {
    Timed t("router_pack", s);
    HIP_TRY(moe::launch_router_pack(b, s));
  }
  if (dW_gate || dbias) {
    Timed t("router_wgrad", s);
    HIP_TRY(moe::launch_router_wgrad(b, s));
  }
  if (dx) {
    Timed t("router_dx", s);
    HIP_TRY(moe::launch_router_dx(b, s));
  }
  g_err.clear();
  return MOE_OK;
}

static int route_common(const Plan& p, const moe_config_t* cfg, const Scores& sc,
                        float* logits_out, int32_t* topk_idx, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* slot, moe_stats_t* stats) {
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  void* ws = cfg->workspace;
  int32_t* idx = topk_idx;
  float* w = topk_w ? topk_w : at<float>(ws, p.w);
  int rc = run_route(p, ws, sc, logits_out, idx, w, s);
  if (rc != MOE_OK) return rc;
  if (counts)
    HIP_TRY(hipMemcpyAsync(counts, at<int32_t>(ws, p.counts), sizeof(int32_t) * p.E,
                           hipMemcpyDeviceToDevice, s));
  if (offsets)
    HIP_TRY(hipMemcpyAsync(offsets, at<int32_t>(ws, p.offsets), sizeof(int32_t) * (p.E + 1),
                           hipMemcpyDeviceToDevice, s));
  if (perm)
    HIP_TRY(hipMemcpyAsync(perm, at<int32_t>(ws, p.perm), sizeof(int32_t) * p.TK,
                           hipMemcpyDeviceToDevice, s));
  if (slot)
    HIP_TRY(hipMemcpyAsync(slot, at<int32_t>(ws, p.slot), sizeof(int32_t) * p.TK,
                           hipMemcpyDeviceToDevice, s));
  if (stats) {
    rc = fill_stats(p, ws, s, stats, at<int32_t>(ws, p.counts), at<int32_t>(ws, p.kcount));
    if (rc != MOE_OK) return rc;
  }
  return MOE_OK;
}

int moe_route(const void* x, const void* W_gate, const moe_config_t* cfg, float* logits,
              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
              int32_t* perm, int32_t* slot, moe_stats_t* stats) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (p.T > 0 && (!x || !W_gate || !topk_idx))
    return fail(MOE_EINVAL, "x, W_gate and topk_idx must be non-NULL");
  if (p.T > 0 && !aligned16({x, W_gate}))
    return fail(MOE_EINVAL, "x and W_gate must be 16-byte aligned");
  rc = check_workspace(cfg, p);
  if (rc != MOE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  if (p.T == 0) {
    if (stats) fill_stats(p, nullptr, s, stats, nullptr, nullptr);
    g_err.clear();
    return MOE_OK;
  }
  rc = arm_canaries(p, cfg->workspace, s);
  if (rc != MOE_OK) return rc;
  Scores sc;
  rc = run_router(p, cfg->workspace, x, W_gate, cfg->logit_bias, s, &sc);
  if (rc != MOE_OK) return rc;
  // the vector router writes finished scores to the workspace; copy them out
  float* lout = logits;
  if (logits && !p.mfma_router)
    HIP_TRY(hipMemcpyAsync(logits, sc.lsrc, sizeof(float) * p.T * p.E,
                           hipMemcpyDeviceToDevice, s));
  if (!p.mfma_router) lout = nullptr;
  rc = route_common(p, cfg, sc, lout, topk_idx, topk_w, counts, offsets, perm, slot, stats);
  if (rc == MOE_OK) g_err.clear();
  return rc;
}

int moe_route_logits(const float* logits, const moe_config_t* cfg, int32_t* topk_idx,
                     float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* slot, moe_stats_t* stats) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (cfg->logit_bias)
    return fail(MOE_EINVAL, "moe_route_logits takes final scores: logit_bias must be NULL");
  if (p.T > 0 && (!logits || !topk_idx))
    return fail(MOE_EINVAL, "logits and topk_idx must be non-NULL");
  rc = check_workspace(cfg, p);
  if (rc != MOE_OK) return rc;
  if (p.T == 0) {
    if (stats) fill_stats(p, nullptr, static_cast<hipStream_t>(cfg->stream), stats, nullptr, nullptr);
    g_err.clear();
    return MOE_OK;
  }
  rc = arm_canaries(p, cfg->workspace, static_cast<hipStream_t>(cfg->stream));
  if (rc != MOE_OK) return rc;
  rc = route_common(p, cfg, Scores{logits, 1, 0, nullptr}, nullptr, topk_idx, topk_w, counts,
                    offsets, perm, slot, stats);
  if (rc == MOE_OK) g_err.clear();
  return rc;
}

int moe_aux_loss(const float* logits, const int32_t* counts, const moe_config_t* cfg,
                 double* aux_out) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (!aux_out) return fail(MOE_EINVAL, "aux_out must be non-NULL");
  if (p.T == 0) {
    *aux_out = 0.0;
    g_err.clear();
    return MOE_OK;
  }
  if (!logits || !counts) return fail(MOE_EINVAL, "logits and counts must be non-NULL");
  rc = check_workspace(cfg, p);
  if (rc != MOE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  void* ws = cfg->workspace;
  rc = arm_canaries(p, ws, s);
  if (rc != MOE_OK) return rc;
  {
    Timed t("softmax_stats", s);
    HIP_TRY(moe::launch_topk_gate(logits, 1, 0, nullptr, nullptr, p.T, p.E, 1, p.gating,
                                  p.renorm, nullptr, nullptr, at<float>(ws, p.ppart),
                                  at<float>(ws, p.hpart), p.topk_blocks, p.topk_tpb, s));
  }
  {
    Timed t("stats", s);
    HIP_TRY(moe::launch_stats(at<float>(ws, p.ppart), at<float>(ws, p.hpart), p.topk_blocks,
                              counts, nullptr, p.T, p.k, p.E, at<double>(ws, p.stats), s));
  }
  double v = 0.0;
  HIP_TRY(hipMemcpyAsync(&v, at<double>(ws, p.stats), sizeof(double), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  *aux_out = v;
  g_err.clear();
  return MOE_OK;
}

int moe_packed_weight_bytes(const moe_config_t* cfg, size_t* w13_bytes, size_t* w2_bytes) {
  int rc = check(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->dtype != MOE_DTYPE_BF16) return fail(MOE_EUNSUPPORTED, "packed weights are for bf16 layers");
  const int64_t n = cfg->n_experts + cfg->n_shared;
  if (w13_bytes)
    *w13_bytes = static_cast<size_t>(2 * n * cfg->d_model * pad_to(cfg->d_ff, kPackW13));
  if (w2_bytes)
    *w2_bytes = static_cast<size_t>(2 * n * cfg->d_ff * pad_to(cfg->d_model, kPackW2));
  g_err.clear();
  return MOE_OK;
}

int moe_pack_weights(const void* W1, const void* W3, const void* W2, const moe_config_t* cfg,
                     void* W1p, void* W3p, void* W2p) {
  int rc = check(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->dtype != MOE_DTYPE_BF16) return fail(MOE_EUNSUPPORTED, "packed weights are for bf16 layers");
  if (!W1 || !W3 || !W2 || !W1p || !W3p || !W2p)
    return fail(MOE_EINVAL, "W1, W3, W2, W1p, W3p and W2p must be non-NULL");
  if (!aligned16({W1, W3, W2, W1p, W3p, W2p}))
    return fail(MOE_EINVAL, "W1, W3, W2, W1p, W3p and W2p must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  const int64_t n = cfg->n_experts + cfg->n_shared;
  HIP_TRY(moe::launch_pack_blocks(W1, n, cfg->d_model, cfg->d_ff, kPackW13, W1p, s));
  HIP_TRY(moe::launch_pack_blocks(W3, n, cfg->d_model, cfg->d_ff, kPackW13, W3p, s));
  HIP_TRY(moe::launch_pack_blocks(W2, n, cfg->d_ff, cfg->d_model, kPackW2, W2p, s));
  g_err.clear();
  return MOE_OK;
}

int moe_debug_canaries(int enable) {
  g_canaries.store(enable != 0, std::memory_order_relaxed);
  return MOE_OK;
}

int moe_debug_check(const moe_config_t* cfg) {
  Plan p;
  int rc = make_plan(cfg, &p);
  if (rc != MOE_OK) return rc;
  if (p.nguards == 0) {
    g_err.clear();
    return 0;
  }
  rc = check_workspace(cfg, p);
  if (rc != MOE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  HIP_TRY(hipStreamSynchronize(s));
  unsigned char buf[kCanaryBytes];
  int bad = 0;
  const char* first = nullptr;
  for (int i = 0; i < p.nguards; ++i) {
    HIP_TRY(hipMemcpy(buf, static_cast<const char*>(cfg->workspace) + p.guard_off[i], kCanaryBytes,
                      hipMemcpyDeviceToHost));
    for (size_t j = 0; j < kCanaryBytes; ++j) {
      if (buf[j] != kCanaryByte) {
        if (!first) first = p.guard_name[i];
        ++bad;
        break;
      }
    }
  }
  if (bad) {
    fail(MOE_OK, "%d workspace guard(s) overwritten; the first after region '%s'", bad, first);
    return bad;
  }
  g_err.clear();
  return 0;
}

double moe_entropy_coef(int64_t step, int64_t total_steps, double high, double low) {
  if (!isfinite(high) || !isfinite(low)) return NAN;
  if (total_steps <= 1) return low;
  const int64_t s = step < 0 ? 0 : (step > total_steps - 1 ? total_steps - 1 : step);
  return high + (low - high) * (static_cast<double>(s) / static_cast<double>(total_steps - 1));
}

int moe_lb_trend(const double* values, int64_t n, double* slope, double* mean) {
  if (!values || !slope || !mean) return fail(MOE_EINVAL, "values, slope and mean must be non-NULL");
  if (n < 2) return fail(MOE_EINVAL, "a trend needs at least 2 values (got %lld)", (long long)n);
  double sum = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite(values[i])) return fail(MOE_EINVAL, "value %lld is not finite", (long long)i);
    sum += values[i];
  }
  const double vm = sum / static_cast<double>(n);
  const double im = static_cast<double>(n - 1) / 2.0;
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double di = static_cast<double>(i) - im;
    num += di * (values[i] - vm);
    den += di * di;
  }
  *slope = num / den;
  *mean = vm;
  g_err.clear();
  return MOE_OK;
}

int moe_timing_enable(int enable) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.enabled = enable != 0;
  return MOE_OK;
}

int moe_timing_only(const char* names) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.only.clear();
  if (!names) return MOE_OK;
  std::string cur;
  for (const char* c = names;; ++c) {
    if (*c == ',' || *c == '\0') {
      if (!cur.empty()) t.only.push_back(cur);
      cur.clear();
      if (*c == '\0') break;
    } else {
      cur.push_back(*c);
    }
  }
  return MOE_OK;
}

int moe_timing_reset(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& l : t.pending) {
    hipEventSynchronize(l.stop);
    t.free_events.push_back(l.start);
    t.free_events.push_back(l.stop);
  }
  t.pending.clear();
  t.names.clear();
  t.launches.clear();
  t.total_ms.clear();
  return MOE_OK;
}

int moe_timing_read(char* names, int64_t* launches, double* total_ms, int max) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& l : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(l.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, l.start, l.stop) == hipSuccess) {
      size_t i = 0;
      for (; i < t.names.size(); ++i)
        if (t.names[i] == l.name) break;
      if (i == t.names.size()) {
        t.names.push_back(l.name);
        t.launches.push_back(0);
        t.total_ms.push_back(0.0);
      }
      t.launches[i] += 1;
      t.total_ms[i] += ms;
    }
    t.free_events.push_back(l.start);
    t.free_events.push_back(l.stop);
  }
  t.pending.clear();
  const int n = static_cast<int>(t.names.size());
  for (int i = 0; i < n && i < max; ++i) {
    if (names) {
      strncpy(names + 64 * i, t.names[i].c_str(), 63);
      names[64 * i + 63] = '\0';
    }
    if (launches) launches[i] = t.launches[i];
    if (total_ms) total_ms[i] = t.total_ms[i];
  }
  return n;
}

}  // extern "C"
