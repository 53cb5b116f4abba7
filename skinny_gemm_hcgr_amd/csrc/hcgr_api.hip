// hcgr_api.hip -- C ABI of the HCGR op (declarations and contract in
// include/hcgr.h). Host code only: argument checks, planning, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/hcgr.h"
#include "hcgr_internal.h"

struct hcgr_op {
  hcgr::Shape shape;
  hcgr_config cfg;
  int device;
  int cu_count;
  std::vector<hcgr::TableEntry> table;  // tuned plans (empty: the heuristic)
  int wait_polls = hcgr::kDefaultWaitPolls;  // hcgr_set_wait_polls
};
static_assert(HCGR_DEFAULT_WAIT_POLLS == hcgr::kDefaultWaitPolls && HCGR_MAX_WAIT_POLLS == hcgr::kMaxWaitPolls,
              "the header's poll budgets are the library's");

// Scratch for hcgr_forward_noalloc: the workspace of callers that cannot
// allocate. Each GPU the library runs on holds one copy until the process
// ends; every call on that GPU shares it.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Device address of each GPU's copy of `scratch`, looked up once per device
// (the host-side name of the array is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

thread_local char g_err[512] = "";

hcgr_status fail(hcgr_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hcgr_status fail(hcgr_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

hcgr_status ok() {
  g_err[0] = '\0';
  return HCGR_OK;
}

// Config checks shared by create, validate and the size queries.
hcgr_status check_config(const hcgr_config* c, hcgr::Shape* out) {
  if (!c) return fail(HCGR_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->hc < 1 || c->hs < 1 || c->r < 1)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "hc, hs and r must be positive (hc=%d hs=%d r=%d)", c->hc, c->hs, c->r);
  if (!std::isfinite(c->eps) || c->eps < 0.0f)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (c->weight_layout != HCGR_WEIGHTS_SEPARATE && c->weight_layout != HCGR_WEIGHTS_MERGED_FOLDED)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "unknown weight_layout %d", c->weight_layout);
  const int64_t k = (int64_t)c->hc * c->hs;
  if (c->wnorm_len != c->hs && (int64_t)c->wnorm_len != k)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "wnorm_len must be hs (%d) or hc*hs (%lld), got %d", c->hs,
                (long long)k, c->wnorm_len);
  if (c->weight_layout == HCGR_WEIGHTS_MERGED_FOLDED && c->n_pad < c->r + c->hc)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "n_pad (%d) must be >= r + hc (%d)", c->n_pad, c->r + c->hc);
  if (c->hc != 1 && c->hc != 2 && c->hc != 4 && c->hc != 8)
    return fail(HCGR_ERR_UNSUPPORTED, "hc=%d: the kernels support hc = 1, 2, 4 or 8", c->hc);
  if (c->hs % 128 != 0 || c->hs > 65536)
    return fail(HCGR_ERR_UNSUPPORTED, "hs=%d: the kernels support multiples of 128 up to 65536", c->hs);
  if (c->r % 32 != 0 || c->r > 512)
    return fail(HCGR_ERR_UNSUPPORTED, "r=%d: the kernels support multiples of 32 up to 512", c->r);
  if (out) {
    out->hc = c->hc;
    out->hs = c->hs;
    out->r = c->r;
    out->eps = c->eps;
    out->wn_full = (int64_t)c->wnorm_len == k && c->wnorm_len != c->hs;
    out->merged = c->weight_layout == HCGR_WEIGHTS_MERGED_FOLDED;
    out->n_pad = c->n_pad;
  }
  return HCGR_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* name;
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

struct PtrCheck {
  const void* p;
  const char* name;
  size_t align;
};

hcgr_status check_ptrs(const PtrCheck* ptrs, int n) {
  for (int i = 0; i < n; ++i) {
    const PtrCheck& p = ptrs[i];
    if (!p.p) return fail(HCGR_ERR_INVALID_ARGUMENT, "%s is NULL", p.name);
    if ((uintptr_t)p.p % p.align) return fail(HCGR_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", p.name, p.align);
  }
  return HCGR_OK;
}

// Checks of the whole op (mix = false) or of the mix entry point (mix =
// true: y, inj and R2 are not part of the call and must be NULL).
hcgr_status check_forward(const hcgr_config* cfg, const hcgr::Shape& s, const uint16_t* R, const uint16_t* y,
                          const uint16_t* inj, int64_t ld_inj, const uint16_t* wnorm, const uint16_t* wd,
                          const uint16_t* wi, const uint16_t* wu, int64_t M, const void* R2, const float* rrms,
                          const void* inj_next, int64_t ld_inj_next, const void* x, const void* ws,
                          size_t ws_bytes, hcgr::Plan* plan_out, bool mix = false,
                          const hcgr::TableEntry* table = nullptr, int ntable = 0) {
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  if (M > (int64_t)1 << 31) return fail(HCGR_ERR_UNSUPPORTED, "M=%lld exceeds 2^31", (long long)M);
  if (M == 0) return ok();
  const bool merged = s.merged;
  const PtrCheck common[] = {{R, "R", 16},    {wnorm, "wnorm", 16}, {wd, "wd", 16},          {wu, "wu", 16},
                             {rrms, "rrms", 4}, {inj_next, "inj_next", 2}, {x, "x", 16}};
  hcgr_status pst = check_ptrs(common, sizeof common / sizeof common[0]);
  if (pst != HCGR_OK) return pst;
  if (mix) {
    if (y || inj || R2) return fail(HCGR_ERR_INVALID_ARGUMENT, "mix takes no y, inj or R2");
  } else {
    const PtrCheck comb[] = {{y, "y", 16}, {inj, "inj", 2}, {R2, "R2", 16}};
    if ((pst = check_ptrs(comb, 3)) != HCGR_OK) return pst;
  }
  if (merged && wi) return fail(HCGR_ERR_INVALID_ARGUMENT, "wi must be NULL with the merged/folded layout");
  if (!merged) {
    if (!wi) return fail(HCGR_ERR_INVALID_ARGUMENT, "wi is NULL");
    if ((uintptr_t)wi % 16) return fail(HCGR_ERR_INVALID_ARGUMENT, "wi is not 16-byte aligned");
  }
  if (!mix && ld_inj < s.hc) return fail(HCGR_ERR_INVALID_ARGUMENT, "ld_inj=%lld < hc=%d", (long long)ld_inj, s.hc);
  if (ld_inj_next < s.hc)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "ld_inj_next=%lld < hc=%d", (long long)ld_inj_next, s.hc);
  hcgr::Plan plan = hcgr::plan_for(s, M, table, ntable);
  if (ws_bytes < plan.ws_bytes)
    return fail(HCGR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed for M=%lld", ws_bytes,
                plan.ws_bytes, (long long)M);
  if (!ws) return fail(HCGR_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if ((uintptr_t)ws % 16) return fail(HCGR_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");

  const uint64_t K = (uint64_t)s.k(), HS = (uint64_t)s.hs, HC = (uint64_t)s.hc, r = (uint64_t)s.r;
  const uint64_t m = (uint64_t)M;
  auto rng = [](const void* p, uint64_t bytes, const char* n) {
    return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes, n};
  };
  const uint64_t wrows = merged ? (uint64_t)s.n_pad : r;
  const Range ins[] = {
      rng(R, m * K * 2, "R"),
      rng(y, mix ? 0 : m * HS * 2, "y"),
      rng(inj, mix ? 0 : ((m - 1) * (uint64_t)ld_inj + HC) * 2, "inj"),
      rng(wnorm, (uint64_t)cfg->wnorm_len * 2, "wnorm"),
      rng(wd, wrows * K * 2, "wd"),
      rng(merged ? nullptr : wi, merged ? 0 : HC * K * 2, "wi"),
      rng(wu, K * r * 2, "wu"),
  };
  const Range outs[] = {
      rng(R2, mix ? 0 : m * K * 2, "R2"),
      rng(rrms, m * HC * 4, "rrms"),
      rng(inj_next, ((m - 1) * (uint64_t)ld_inj_next + HC) * 2, "inj_next"),
      rng(x, m * HS * 2, "x"),
      rng(ws, plan.ws_bytes, "workspace"),
  };
  const int nin = sizeof ins / sizeof ins[0], nout = sizeof outs / sizeof outs[0];
  for (int i = 0; i < nout; ++i) {
    if (outs[i].hi == outs[i].lo) continue;  // not part of this call
    for (int j = i + 1; j < nout; ++j)
      if (outs[j].hi > outs[j].lo && overlap(outs[i], outs[j]))
        return fail(HCGR_ERR_ALIASING, "output %s overlaps output %s", outs[i].name, outs[j].name);
    for (int j = 0; j < nin; ++j)
      if (ins[j].hi > ins[j].lo && overlap(outs[i], ins[j]))
        return fail(HCGR_ERR_ALIASING, "output %s overlaps input %s", outs[i].name, ins[j].name);
  }
  if (plan_out) *plan_out = plan;
  return ok();
}

// A C ABI plan choice as the planner's Choice; false for an unknown kind.
bool to_choice(const hcgr_plan_choice& c, hcgr::Choice* out) {
  hcgr::Choice x;
  x.kind = c.kind;
  x.kd = c.down_variant;
  x.spw = c.streams_per_wg;
  x.nseg = c.segments;
  x.kt = c.up_variant;  // 0 staged, 1 sweep, 2 generic, 3 generic over 128 tokens, 4 sweep over 256: KT_* values
  x.nranges = c.ranges;
  if (c.kind != HCGR_PLAN_HEURISTIC && c.kind != HCGR_PLAN_SPLIT && c.kind != HCGR_PLAN_TILE &&
      c.kind != HCGR_PLAN_FUSED && c.kind != HCGR_PLAN_PERSISTENT)
    return false;
  *out = x;
  return true;
}

hcgr_plan_choice from_choice(const hcgr::Choice& c, int64_t tokens) {
  hcgr_plan_choice o;
  o.tokens = tokens;
  o.kind = c.kind;
  o.down_variant = c.kind == HCGR_PLAN_HEURISTIC ? 0 : c.kd;
  o.streams_per_wg = c.kind == HCGR_PLAN_TILE ? c.spw : 0;
  o.segments = c.kind == HCGR_PLAN_TILE ? c.nseg : 0;
  o.up_variant = c.kind == HCGR_PLAN_TILE ? c.kt : 0;
  o.ranges = c.kind == HCGR_PLAN_TILE ? c.nranges : 0;
  return o;
}

// Checks a C ABI table against a shape and converts it.
hcgr_status check_table(const hcgr::Shape& s, const hcgr_plan_choice* t, int32_t n, std::vector<hcgr::TableEntry>* out) {
  if (n < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "table length %d is negative", n);
  if (n > 0 && !t) return fail(HCGR_ERR_INVALID_ARGUMENT, "table is NULL");
  std::vector<hcgr::TableEntry> v;
  v.reserve((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    hcgr::Choice c;
    if (!to_choice(t[i], &c)) return fail(HCGR_ERR_INVALID_ARGUMENT, "table entry %d: unknown kind %d", i, t[i].kind);
    if (t[i].tokens < 1 || (i > 0 && t[i].tokens <= t[i - 1].tokens))
      return fail(HCGR_ERR_INVALID_ARGUMENT, "table entry %d: keys must be >= 1 and strictly increasing", i);
    hcgr::Plan p;
    if (c.kind != hcgr::kChoiceHeuristic && !hcgr::plan_from_choice(s, t[i].tokens, c, &p))
      return fail(HCGR_ERR_INVALID_ARGUMENT, "table entry %d (tokens=%lld): the choice cannot run this shape", i,
                  (long long)t[i].tokens);
    v.push_back(hcgr::TableEntry{t[i].tokens, c});
  }
  *out = std::move(v);
  return HCGR_OK;
}

}  // namespace

extern "C" {

const char* hcgr_status_string(hcgr_status s) {
  switch (s) {
    case HCGR_OK: return "HCGR_OK";
    case HCGR_ERR_INVALID_ARGUMENT: return "HCGR_ERR_INVALID_ARGUMENT";
    case HCGR_ERR_UNSUPPORTED: return "HCGR_ERR_UNSUPPORTED";
    case HCGR_ERR_ALIASING: return "HCGR_ERR_ALIASING";
    case HCGR_ERR_WORKSPACE_TOO_SMALL: return "HCGR_ERR_WORKSPACE_TOO_SMALL";
    case HCGR_ERR_HIP: return "HCGR_ERR_HIP";
  }
  return "HCGR_ERR_UNKNOWN";
}

const char* hcgr_last_error(void) { return g_err; }

hcgr_status hcgr_workspace_size_for(const hcgr_config* cfg, int64_t M, size_t* bytes) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  if (!bytes) return fail(HCGR_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  *bytes = hcgr::workspace_bound(s, M);
  return ok();
}

static const char* k2_name(int kt) {
  return kt == hcgr::KT_SWEEP2 ? "k2_sweep2" : kt == hcgr::KT_SWEEP ? "k2_sweep" : hcgr::is_gen(kt) ? "k2_gen" : "k2_stage";
}
static long long k2_grid(const hcgr::Shape& s, const hcgr::Plan& p, int64_t M) {
  const hcgr::KTShape t = hcgr::kt_shape(p.kt);
  if (hcgr::is_gen(p.kt)) return (long long)(hcgr::cdiv(M, t.tm) * (s.hs / t.cb));
  if (hcgr::is_sweep(p.kt)) return (long long)(hcgr::cdiv(M, t.tm) * p.nranges);
  return (long long)(hcgr::cdiv(hcgr::cdiv(M, t.tm) * (s.hs / 64), 8) * 16);
}

static void describe(const hcgr::Shape& s, const hcgr::Plan& p, int64_t M, char* buf, size_t len) {
  if (len) {
    if (M == 0) {
      snprintf(buf, len, "M=0: no launch");
    } else if (p.kind == hcgr::PLAN_FUSED) {
      snprintf(buf, len,
               "M=%lld plan=fused mpad=%lld | k1_fuse tm=%d row_blocks=1 chunks=%d (%d per stream) tiles=%d grid=%dx%d "
               "last-arrival reduction | k2_decg tm=%d waves=%d channels=%d grid=%dx%d | workspace=%zu",
               (long long)M, (long long)p.mpad, p.tm, p.nkc, p.kcps, p.ntiles, s.nblk() * p.nkc, p.ntiles, p.tm, p.upw,
               p.cb, s.hs / p.cb, p.ntiles, p.ws_bytes);
    } else if (p.kind == hcgr::PLAN_PERSIST) {
      snprintf(buf, len,
               "M=%lld plan=persistent mpad=%lld | dec_persist tm=%d one kernel: down role row_blocks=1 chunks=%d "
               "(%d per stream) tiles=%d workgroups=%d, last-arrival reduction; up role waves=4 channels=%d "
               "workgroups=%d, waits for the tile's h | workspace=%zu",
               (long long)M, (long long)p.mpad, p.tm, p.nkc, p.kcps, p.ntiles, s.nblk() * p.nkc * p.ntiles, p.cb,
               s.hs / p.cb * p.ntiles, p.ws_bytes);
    } else if (p.kind == hcgr::PLAN_SPLIT) {
      hcgr::KDShape a = hcgr::kd_shape(p.k1);
      hcgr::K2Shape b = hcgr::k2_shape(p.k2);
      snprintf(buf, len,
               "M=%lld plan=split mpad=%lld | k1_dec tm=%d row_blocks=%d k_waves=%d k_chunk=%d chunks=%d n_tiles=%d "
               "grid=%dx%lld | k1_reduce waves=%lld | %s tm=%d waves=%d channels=%d grid=%dx%lld | "
               "workspace=%zu",
               (long long)M, (long long)p.mpad, a.tm, a.rb, a.kw, p.kc, p.nkc, p.ntiles_n, p.ntiles_n * p.nkc,
               (long long)(p.mpad / p.tm), (long long)(s.n_rows() * (p.mpad / 16)), s.hc == 4 ? "k2_dec" : "k2_decg",
               b.tm, s.hc == 4 ? (p.cb + 3) / 4 : hcgr::decg_waves(s.hc, s.hs), p.cb, s.hs / p.cb,
               (long long)hcgr::cdiv(M, (int64_t)b.tm), p.ws_bytes);
    } else if (p.kind == hcgr::PLAN_TILE) {
      hcgr::KTShape t = hcgr::kt_shape(p.kt);
      snprintf(buf, len,
               "M=%lld plan=tile | k1_tile tm=%d waves=8 stage_k=64 streams/wg=%d row_splits=%d segments=%d%s grid=%lld%s | "
               "%s tm=%d channels=%d ranges=%d grid=%lld | workspace=%zu",
               (long long)M, p.tm, p.spw, p.nsplit, p.nseg, p.xgroup ? " tile_xcd" : "",
               (long long)((p.xgroup ? hcgr::cdiv(hcgr::cdiv(M, (int64_t)p.tm), 8) * 8 : hcgr::cdiv(M, (int64_t)p.tm)) *
                           p.nsplit * (s.hc / p.spw) * p.nseg),
               p.spw == 1 ? " | k1_sum" : "",
               k2_name(p.kt), t.tm, t.cb, p.nranges, k2_grid(s, p, M), p.ws_bytes);
    } else {
      hcgr::KFShape f = hcgr::kf_shape(p.kf);
      hcgr::KTShape t = hcgr::kt_shape(p.kt);
      snprintf(buf, len,
               "M=%lld plan=%s | k1_full tm=%d waves=%d stage_k=%d streams/wg=%d row_splits=%d grid=%lldx%d%s | "
               "%s tm=%d channels=%d ranges=%d grid=%lld | workspace=%zu",
               (long long)M, p.kind == hcgr::PLAN_FULL ? "full" : "stream", f.tm, f.nw, f.ks, p.spw, p.nsplit,
               (long long)hcgr::cdiv(M, f.tm), p.nsplit * (4 / p.spw), p.kind == hcgr::PLAN_STREAM ? " | k1_sum" : "",
               k2_name(p.kt), t.tm, t.cb, p.nranges, k2_grid(s, p, M), p.ws_bytes);
    }
  }
}

hcgr_status hcgr_describe_plan(const hcgr_config* cfg, int64_t M, char* buf, size_t len) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  if (!buf && len) return fail(HCGR_ERR_INVALID_ARGUMENT, "buf is NULL");
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  describe(s, hcgr::make_plan(s, M), M, buf, len);
  return ok();
}

hcgr_status hcgr_plan_candidates(const hcgr_config* cfg, int64_t M, hcgr_plan_choice* out, int32_t capacity,
                                 int32_t* count) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  if (!count) return fail(HCGR_ERR_INVALID_ARGUMENT, "count is NULL");
  if (M < 1) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld: candidates need M >= 1", (long long)M);
  if (capacity < 0 || (capacity > 0 && !out)) return fail(HCGR_ERR_INVALID_ARGUMENT, "bad output capacity");
  std::vector<hcgr::Choice> v(512);
  const int n = hcgr::plan_choices(s, M, v.data(), (int)v.size());
  for (int i = 0; i < n && i < capacity && i < (int)v.size(); ++i) out[i] = from_choice(v[(size_t)i], M);
  *count = n;
  return ok();
}

hcgr_status hcgr_plan_lookup(const hcgr_config* cfg, const hcgr_plan_choice* table, int32_t n, int64_t M,
                             hcgr_plan_choice* chosen, char* buf, size_t len) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  if (!buf && len) return fail(HCGR_ERR_INVALID_ARGUMENT, "buf is NULL");
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  std::vector<hcgr::TableEntry> t;
  if ((st = check_table(s, table, n, &t)) != HCGR_OK) return st;
  const int i = hcgr::table_index(t.data(), (int)t.size(), M);
  hcgr::Plan p;
  const bool use = i >= 0 && t[(size_t)i].c.kind != hcgr::kChoiceHeuristic &&
                   hcgr::plan_from_choice(s, M, t[(size_t)i].c, &p);
  if (chosen) *chosen = use ? from_choice(t[(size_t)i].c, t[(size_t)i].M) : from_choice(hcgr::Choice(), i >= 0 ? t[(size_t)i].M : 0);
  if (M == 0) {
    if (len) snprintf(buf, len, "M=0: no launch");
  } else {
    describe(s, use ? p : hcgr::make_plan(s, M), M, buf, len);
  }
  return ok();
}

hcgr_status hcgr_workspace_size_table(const hcgr_config* cfg, const hcgr_plan_choice* table, int32_t n, int64_t M,
                                      size_t* bytes) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  if (!bytes) return fail(HCGR_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  std::vector<hcgr::TableEntry> t;
  if ((st = check_table(s, table, n, &t)) != HCGR_OK) return st;
  *bytes = hcgr::workspace_bound_table(s, M, t.data(), (int)t.size());
  return ok();
}

hcgr_status hcgr_set_plan_table(hcgr_handle h, const hcgr_plan_choice* table, int32_t n) {
  if (!h) return fail(HCGR_ERR_INVALID_ARGUMENT, "handle is NULL");
  std::vector<hcgr::TableEntry> t;
  hcgr_status st = check_table(h->shape, table, n, &t);
  if (st != HCGR_OK) return st;
  h->table = std::move(t);
  return ok();
}

// Looks up the current device's copy of `scratch` and zeroes its counter
// bytes, once per device; `device` must be current.
static hcgr_status scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(HCGR_ERR_UNSUPPORTED, "device %d: at most %d devices", device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return HCGR_OK;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return fail(HCGR_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  if ((e = hipMemset(p, 0, hcgr::kCtrBytes)) != hipSuccess)
    return fail(HCGR_ERR_HIP, "zeroing the scratch counters: %s", hipGetErrorString(e));
  g_scratch[device] = p;
  return HCGR_OK;
}

hcgr_status hcgr_create(const hcgr_config* cfg, int device, hcgr_handle* out) {
  if (!out) return fail(HCGR_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipGetDeviceCount: %s", hipGetErrorString(e));
  if (device < 0 || device >= ndev)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "device %d out of range (%d devices)", device, ndev);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(HCGR_ERR_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950 (MI355X)", device,
                prop.gcnArchName);
  int cur = -1;
  e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
    return fail(HCGR_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(e));
  int ke = hcgr::configure_kernels();
  const hcgr_status sst = ke == (int)hipSuccess ? scratch_setup(device) : HCGR_OK;
  if (cur != device) (void)hipSetDevice(cur);
  if (ke != (int)hipSuccess)
    return fail(HCGR_ERR_HIP, "kernel attribute set-up failed: %s", hipGetErrorString((hipError_t)ke));
  if (sst != HCGR_OK) return sst;
  hcgr_op* op = new (std::nothrow) hcgr_op;
  if (!op) return fail(HCGR_ERR_INVALID_ARGUMENT, "out of host memory");
  op->shape = s;
  op->cfg = *cfg;
  op->device = device;
  op->cu_count = prop.multiProcessorCount;
  *out = op;
  return ok();
}

void hcgr_destroy(hcgr_handle h) { delete h; }

hcgr_status hcgr_set_wait_polls(hcgr_handle h, int32_t polls) {
  if (!h) return fail(HCGR_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (polls < 0 || polls > hcgr::kMaxWaitPolls)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "polls=%d is outside 0..%d", (int)polls, hcgr::kMaxWaitPolls);
  h->wait_polls = polls;
  return ok();
}

hcgr_status hcgr_workspace_size(hcgr_handle h, int64_t M, size_t* bytes) {
  if (!h) return fail(HCGR_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (!bytes) return fail(HCGR_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  *bytes = hcgr::workspace_bound_table(h->shape, M, h->table.data(), (int)h->table.size());
  return ok();
}

hcgr_status hcgr_validate(const hcgr_config* cfg, const uint16_t* R, const uint16_t* y, const uint16_t* inj,
                          int64_t ld_inj, const uint16_t* wnorm, const uint16_t* wd, const uint16_t* wi,
                          const uint16_t* wu, int64_t M, const uint16_t* R2, const float* rrms,
                          const uint16_t* inj_next, int64_t ld_inj_next, const uint16_t* x, const void* workspace,
                          size_t workspace_bytes) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  return check_forward(cfg, s, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x,
                       workspace, workspace_bytes, nullptr);
}

// Stream and device checks shared by every launching entry point; on success
// *prev is the caller's current device (restore it with restore_device).
static hcgr_status enter_device(hcgr_handle h, void* stream, int* prev) {
  int dev = -1;
  hipError_t e;
  if (stream) {
    e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  } else {
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev != h->device)
    return fail(HCGR_ERR_INVALID_ARGUMENT, "stream belongs to device %d, handle to device %d", dev, h->device);
  int cur = -1;
  e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (cur != h->device) {
    e = hipSetDevice(h->device);
    if (e != hipSuccess) return fail(HCGR_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(e));
  }
  *prev = cur;
  return HCGR_OK;
}
static void restore_device(hcgr_handle h, int prev) {
  if (prev != h->device) (void)hipSetDevice(prev);
}

static hcgr_status forward_impl(hcgr_handle h, const uint16_t* R, const uint16_t* y, const uint16_t* inj,
                                int64_t ld_inj, const uint16_t* wnorm, const uint16_t* wd, const uint16_t* wi,
                                const uint16_t* wu, int64_t M, uint16_t* R2, float* rrms, uint16_t* inj_next,
                                int64_t ld_inj_next, uint16_t* x, void* workspace, size_t workspace_bytes,
                                void* stream, void* const* events, bool mix = false) {
  if (!h) return fail(HCGR_ERR_INVALID_ARGUMENT, "handle is NULL");
  hcgr::Plan plan;
  hcgr_status st = check_forward(&h->cfg, h->shape, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next,
                                 ld_inj_next, x, workspace, workspace_bytes, &plan, mix, h->table.data(),
                                 (int)h->table.size());
  if (st != HCGR_OK || M == 0) return st;
  int cur = -1;
  if ((st = enter_device(h, stream, &cur)) != HCGR_OK) return st;
  hcgr::ForwardArgs a;
  a.R = R; a.y = y; a.inj = inj; a.wnorm = wnorm; a.wd = wd; a.wi = wi; a.wu = wu;
  a.ld_inj = ld_inj; a.ld_inj_next = ld_inj_next; a.M = M;
  a.R2 = R2; a.inj_next = inj_next; a.x = x; a.rrms = rrms; a.ws = workspace;
  a.res = mix ? R : R2;
  a.wait_polls = h->wait_polls;
  int le = hcgr::launch_forward(h->shape, plan, a, stream, events);
  restore_device(h, cur);
  if (le != (int)hipSuccess)
    return fail(HCGR_ERR_HIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)le));
  return ok();
}

hcgr_status hcgr_forward(hcgr_handle h, const uint16_t* R, const uint16_t* y, const uint16_t* inj, int64_t ld_inj,
                         const uint16_t* wnorm, const uint16_t* wd, const uint16_t* wi, const uint16_t* wu, int64_t M,
                         uint16_t* R2, float* rrms, uint16_t* inj_next, int64_t ld_inj_next, uint16_t* x,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(h, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x, workspace,
                      workspace_bytes, stream, nullptr);
}

hcgr_status hcgr_forward_noalloc(hcgr_handle h, const uint16_t* R, const uint16_t* y, const uint16_t* inj,
                                 int64_t ld_inj, const uint16_t* wnorm, const uint16_t* wd, const uint16_t* wi,
                                 const uint16_t* wu, int64_t M, uint16_t* R2, float* rrms, uint16_t* inj_next,
                                 int64_t ld_inj_next, uint16_t* x, void* stream) {
  if (!h) return fail(HCGR_ERR_INVALID_ARGUMENT, "handle is NULL");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ws = h->device >= 0 && h->device < kMaxDevices ? g_scratch[h->device] : nullptr;
  }
  if (!ws) return fail(HCGR_ERR_HIP, "no scratch on device %d", h->device);
  if (M > 0) {
    const hcgr::Plan plan = hcgr::plan_for(h->shape, M, h->table.data(), (int)h->table.size());
    if (plan.ws_bytes > kScratchBytes)
      return fail(HCGR_ERR_WORKSPACE_TOO_SMALL,
                  "M=%lld needs %zu bytes of workspace; the library's scratch holds %zu (call hcgr_forward with a "
                  "workspace)",
                  (long long)M, plan.ws_bytes, kScratchBytes);
  }
  return forward_impl(h, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x, ws,
                      kScratchBytes, stream, nullptr);
}

size_t hcgr_noalloc_scratch_bytes(void) { return kScratchBytes; }

hcgr_status hcgr_forward_timed(hcgr_handle h, const uint16_t* R, const uint16_t* y, const uint16_t* inj,
                               int64_t ld_inj, const uint16_t* wnorm, const uint16_t* wd, const uint16_t* wi,
                               const uint16_t* wu, int64_t M, uint16_t* R2, float* rrms, uint16_t* inj_next,
                               int64_t ld_inj_next, uint16_t* x, void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events) {
  if (!events) return fail(HCGR_ERR_INVALID_ARGUMENT, "events is NULL");
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return fail(HCGR_ERR_INVALID_ARGUMENT, "events[%d] is NULL", i);
  return forward_impl(h, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x, workspace,
                      workspace_bytes, stream, events);
}

hcgr_status hcgr_mix(hcgr_handle h, const uint16_t* R, const uint16_t* wnorm, const uint16_t* wd,
                     const uint16_t* wi, const uint16_t* wu, int64_t M, float* rrms, uint16_t* inj_next,
                     int64_t ld_inj_next, uint16_t* x, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(h, R, nullptr, nullptr, 0, wnorm, wd, wi, wu, M, nullptr, rrms, inj_next, ld_inj_next, x,
                      workspace, workspace_bytes, stream, nullptr, true);
}

hcgr_status hcgr_validate_mix(const hcgr_config* cfg, const uint16_t* R, const uint16_t* wnorm, const uint16_t* wd,
                              const uint16_t* wi, const uint16_t* wu, int64_t M, const float* rrms,
                              const uint16_t* inj_next, int64_t ld_inj_next, const uint16_t* x, const void* workspace,
                              size_t workspace_bytes) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  return check_forward(cfg, s, R, nullptr, nullptr, 0, wnorm, wd, wi, wu, M, nullptr, rrms, inj_next, ld_inj_next,
                       x, workspace, workspace_bytes, nullptr, true);
}

hcgr_status hcgr_validate_combine(const hcgr_config* cfg, const uint16_t* R, const uint16_t* y,
                                  const uint16_t* inj, int64_t ld_inj, int64_t M, const uint16_t* R2) {
  hcgr::Shape s;
  hcgr_status st = check_config(cfg, &s);
  if (st != HCGR_OK) return st;
  if (M < 0) return fail(HCGR_ERR_INVALID_ARGUMENT, "M=%lld is negative", (long long)M);
  if (M > (int64_t)1 << 31) return fail(HCGR_ERR_UNSUPPORTED, "M=%lld exceeds 2^31", (long long)M);
  if (M == 0) return ok();
  const PtrCheck ptrs[] = {{R, "R", 16}, {y, "y", 16}, {inj, "inj", 2}, {R2, "R2", 16}};
  if ((st = check_ptrs(ptrs, 4)) != HCGR_OK) return st;
  if (ld_inj < s.hc) return fail(HCGR_ERR_INVALID_ARGUMENT, "ld_inj=%lld < hc=%d", (long long)ld_inj, s.hc);
  const uint64_t m = (uint64_t)M, K = (uint64_t)s.k();
  const Range out{(uintptr_t)R2, (uintptr_t)R2 + (uintptr_t)(m * K * 2), "R2"};
  const Range ins[] = {{(uintptr_t)R, (uintptr_t)R + (uintptr_t)(m * K * 2), "R"},
                       {(uintptr_t)y, (uintptr_t)y + (uintptr_t)(m * (uint64_t)s.hs * 2), "y"},
                       {(uintptr_t)inj, (uintptr_t)inj + (uintptr_t)(((m - 1) * (uint64_t)ld_inj + (uint64_t)s.hc) * 2),
                        "inj"}};
  for (const Range& in : ins)
    if (overlap(out, in)) return fail(HCGR_ERR_ALIASING, "output R2 overlaps input %s", in.name);
  return ok();
}

hcgr_status hcgr_combine(hcgr_handle h, const uint16_t* R, const uint16_t* y, const uint16_t* inj, int64_t ld_inj,
                         int64_t M, uint16_t* R2, void* stream) {
  if (!h) return fail(HCGR_ERR_INVALID_ARGUMENT, "handle is NULL");
  hcgr_status st = hcgr_validate_combine(&h->cfg, R, y, inj, ld_inj, M, R2);
  if (st != HCGR_OK || M == 0) return st;
  int cur = -1;
  if ((st = enter_device(h, stream, &cur)) != HCGR_OK) return st;
  hcgr::CombineArgs a;
  a.R = R; a.y = y; a.inj = inj; a.ld_inj = ld_inj; a.M = M; a.HS = h->shape.hs; a.HC = h->shape.hc; a.R2 = R2;
  int le = hcgr::launch_combine(a, stream);
  restore_device(h, cur);
  if (le != (int)hipSuccess)
    return fail(HCGR_ERR_HIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)le));
  return ok();
}

}  // extern "C"
