// C ABI of the EXL3 layer: argument validation, workspace layout, path choice and launches.
// Host work only; every step of the layer runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/exl3.h"
#include "exl3_internal.hpp"

using namespace exl3;

namespace exl3 {
// the dense MLP block's down input from its gate_up output (k_prepass.hip): h = bf16(silu(g) * u) rotated into the
// fragment-major fp16 operand of launch_prepass_f16.
hipError_t launch_prepass_silu_f16(const void* gu, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                                   hipStream_t stream, bool rows32 = false);
}  // namespace exl3

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return EXL3_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(EXL3_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return EXL3_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr unsigned kKnownFlags =
    EXL3_ACT_INT8 | EXL3_FORCE_GEMV | EXL3_FORCE_MFMA | EXL3_GEMM_NO_SPLIT | EXL3_BATCH_INVARIANT;
// The GEMM runs unsplit under either flag.
constexpr unsigned kNoSplitFlags = EXL3_GEMM_NO_SPLIT | EXL3_BATCH_INVARIANT;
// Dispatch threshold.  The decode-phase path streams every weight once per 16-row launch, so its time
// grows with ceil(M/16) * OC; the MFMA GEMM splits the input features of a shard with few output tiles
// so that about 1024 waves run, which keeps its time nearly flat in M up to a few hundred rows.
// Measured over the projections of a 5120/17408 decoder (M sweep, 64 layers) the decode path is faster
// up to 32 rows for 17408 and 7168 outputs and up to 48 for 5120; the threshold
// 16 * clamp(16384 / OC, 2, 8) follows that, between two and eight launches.
int64_t gemv_max_rows(int64_t OC) {
  int64_t chunks = OC > 0 ? 10240 / OC : 2;
  chunks = chunks < 2 ? 2 : (chunks > 8 ? 8 : chunks);
  return chunks * kDecodeMaxRows;
}

int check_flags(unsigned flags) {
  if (flags & ~kKnownFlags) return fail(EXL3_EINVAL, "flags: unknown bits 0x%x", flags & ~kKnownFlags);
  if ((flags & EXL3_FORCE_GEMV) && (flags & EXL3_FORCE_MFMA))
    return fail(EXL3_EINVAL, "flags: EXL3_FORCE_GEMV and EXL3_FORCE_MFMA are exclusive");
  if ((flags & EXL3_BATCH_INVARIANT) && (flags & EXL3_FORCE_MFMA))
    return fail(EXL3_EINVAL, "flags: EXL3_BATCH_INVARIANT selects the decode-phase kernel; EXL3_FORCE_MFMA cannot be combined with it");
  return EXL3_OK;
}

int check_dims(int64_t M, int64_t IC) {
  if (M < 0) return fail(EXL3_EINVAL, "M: %lld is negative", (long long)M);
  if (M > (int64_t(1) << 30)) return fail(EXL3_EINVAL, "M: %lld is too large", (long long)M);
  if (IC <= 0 || IC % 128) return fail(EXL3_EINVAL, "IC: %lld is not a positive multiple of 128", (long long)IC);
  if (IC > (int64_t(1) << 20)) return fail(EXL3_EINVAL, "IC: %lld is too large", (long long)IC);
  return EXL3_OK;
}

int check_shard(const char* who, int64_t IC, const int16_t* code, int64_t OC, int K, int64_t col0, int64_t ldo,
                const void* s_in, const void* rin, const void* rout, const void* s_out) {
  if (OC <= 0 || OC % 128) return fail(EXL3_EINVAL, "%sOC: %lld is not a positive multiple of 128", who, (long long)OC);
  if (OC / 128 > kCounterSlots) return fail(EXL3_EINVAL, "%sOC: %lld exceeds %d blocks of 128", who, (long long)OC, kCounterSlots);
  if (K < 1 || K > 8) return fail(EXL3_EINVAL, "%sK: %d is outside 1..8", who, K);
  if (col0 < 0 || col0 + OC > ldo)
    return fail(EXL3_EINVAL, "%scol0: slice [%lld, %lld) does not fit ldo %lld", who, (long long)col0,
                (long long)(col0 + OC), (long long)ldo);
  if (IC / 16 * (OC / 16) * 32 * int64_t(K) >= (int64_t(1) << 31))
    return fail(EXL3_EUNSUPPORTED, "%scode: %lld x %lld at K=%d exceeds 2 GiB of trellis words per shard", who,
                (long long)IC, (long long)OC, K);
  if (!code) return fail(EXL3_EINVAL, "%scode: null", who);
  if (!aligned(code, 16)) return fail(EXL3_EINVAL, "%scode: not 16-byte aligned", who);
  if (!s_in || !rin) return fail(EXL3_EINVAL, "%ss_in/rin: null", who);
  if (!aligned(s_in, 4) || !aligned(rin, 4)) return fail(EXL3_EINVAL, "%ss_in/rin: not 4-byte aligned", who);
  if (!rout || !s_out) return fail(EXL3_EINVAL, "%srout/s_out: null", who);
  if (!aligned(rout, 2) || !aligned(s_out, 2)) return fail(EXL3_EINVAL, "%srout/s_out: not 2-byte aligned", who);
  (void)IC;
  return EXL3_OK;
}

// The prefill/decode choice is made here, inside the op, by M ("radiance_escha.py", `escha_linear_into`: the
// 8-bit staging buffers serve either phase).  With EXL3_BATCH_INVARIANT the 8-bit path keeps the unsplit GEMM,
// whose order per output does not depend on M.
bool use_decode_path(int64_t M, unsigned flags, int64_t OC) {
  if ((flags & EXL3_ACT_INT8) && (flags & EXL3_BATCH_INVARIANT)) return false;
  if (flags & (EXL3_FORCE_GEMV | EXL3_BATCH_INVARIANT)) return true;
  if (flags & EXL3_FORCE_MFMA) return false;
  return M <= gemv_max_rows(OC);
}

// Row chunks the decode-phase path launches: full chunks of kDecodeLaunchRows rows, then the remainder.
int64_t first_chunk(int64_t M) { return M < kDecodeLaunchRows ? M : kDecodeLaunchRows; }
int64_t last_chunk(int64_t M) { return M - (M - 1) / kDecodeLaunchRows * kDecodeLaunchRows; }
// Rows the pre-rotation region of a decode-phase call holds: its largest chunk, padded to 16-row fragments.
int64_t pre_rows(int64_t M) { return (first_chunk(M) + kDecodeMaxRows - 1) / kDecodeMaxRows * kDecodeMaxRows; }

// Slab bytes the decode-phase path needs for these shards (mixes the kernels do not cover run one
// launch per shard); false if some chunk cannot be planned.
bool decode_slab_bytes(int64_t M, int64_t IC, int n, const DecShardIn* in, size_t* need, bool pre) {
  *need = 0;
  for (int64_t rows : {first_chunk(M), last_chunk(M)}) {
    DecPlan pl;
    if (!plan_decode(rows, IC, n, in, &pl, pre)) return false;
    if (pl.kset < 0) {
      for (int i = 0; i < n; ++i) {
        DecPlan p1;
        if (!plan_decode(rows, IC, 1, in + i, &p1, pre)) return false;
        *need = p1.slab_bytes > *need ? p1.slab_bytes : *need;
      }
    } else {
      *need = pl.slab_bytes > *need ? pl.slab_bytes : *need;
    }
  }
  return true;
}

struct Layout {
  size_t slab_off, slab_bytes;   // split-K slab: decode-phase partials, or the prefill GEMM's partial tiles
  size_t xh_off, xh_bytes;       // prefill-phase rotated activations, one region per distinct (s_in, rin)
  size_t scale_off;              // 8-bit path: the row scales, at this offset inside each region
  size_t part_off;               // 8-bit path: per-(row, 128-block) max |xh|, at this offset inside each region
  size_t total;
};

// rows_pad: the rotated activations' rows are padded to a multiple of this (16-row fragments for the
// decode-phase kernel, 32-row ones for the prefill GEMM).
Layout layout_for(size_t slab_bytes, int64_t M = 0, int64_t IC = 0, int n_xh = 0, bool int8 = false,
                  int64_t rows_pad = 32) {
  Layout L;
  L.slab_off = align_up(kCounterBytes);
  L.slab_bytes = align_up(slab_bytes);
  L.xh_off = L.slab_off + L.slab_bytes;
  L.scale_off = align_up(size_t((M + rows_pad - 1) / rows_pad * rows_pad) * size_t(IC) * 2);
  L.part_off = L.scale_off + (int8 ? align_up(size_t(M) * 4) : 0);
  L.xh_bytes = L.part_off + (int8 ? align_up(size_t(M) * size_t(IC / 128) * 4) : 0);
  L.total = L.xh_off + L.xh_bytes * size_t(n_xh);
  return L;
}

// Distinct (s_in, rin) pairs among the shards, in first-use order; slot[i] = region of shard i.
int distinct_inputs(int n, const DecShardIn* in, int* slot) {
  int k = 0;
  for (int i = 0; i < n; ++i) {
    slot[i] = -1;
    for (int j = 0; j < i; ++j)
      if (in[j].s_in == in[i].s_in && in[j].rin == in[i].rin) { slot[i] = slot[j]; break; }
    if (slot[i] < 0) slot[i] = k++;
  }
  return k;
}

int check_workspace(const Layout& L, void* ws, size_t ws_bytes) {
  if (!ws) return fail(EXL3_EWORKSPACE, "ws: null (need %zu bytes)", L.total);
  if (!aligned(ws, kAlign)) return fail(EXL3_EINVAL, "ws: not %zu-byte aligned", kAlign);
  if (ws_bytes < L.total) return fail(EXL3_EWORKSPACE, "ws_bytes: %zu < required %zu", ws_bytes, L.total);
  return EXL3_OK;
}

// The decode-phase path: one launch per chunk of <= 32 rows covering every shard.  A chunk of at least
// kPreRotateRows rows first rotates its activations once per distinct (s_in, rin) into the workspace
// (fragment-major, 16-row blocks), and the decode launch reads them from there (a chunk of 17..32 rows
// as two 16-row groups in one launch, so the weights are streamed once per 32 rows).
// gu (optional): the dense MLP block's gate_up output [M, 2 IC]; the pre-rotation (5..32 rows) or the decode
// kernel's in-block pre-pass (1..4 rows) then forms the input h = bf16(silu(g) * u) itself.
// int8: the 8-bit path.  A chunk of 5..32 rows first writes its integer codes (as fp16 numbers) and row
// scales with the fragment-major 8-bit pre-pass; a chunk of 1..4 rows only the per-(row, block) maxima, and
// the decode kernel's in-block pre-pass forms the same codes.  The decode launch multiplies the codes and
// applies each row's scale after its output Hadamard, as the GEMM's epilogue does.
int run_decode(const char* who, void* out, int64_t ldo, const void* x, int64_t M, int64_t IC, int n,
               const DecShardIn* in_, char* ws, const Layout& L, hipStream_t stream, const void* gu = nullptr,
               bool int8 = false) {
  if (int8 && gu) return fail(EXL3_EUNSUPPORTED, "%s: the folded activation is for the 16-bit path", who);
  DecShardIn in[kMaxShards];
  for (int i = 0; i < n; ++i) in[i] = in_[i];
  int slot[kMaxShards];
  distinct_inputs(n, in, slot);
  for (int64_t r0 = 0; r0 < M; r0 += kDecodeLaunchRows) {
    const int64_t rows = (M - r0) < kDecodeLaunchRows ? (M - r0) : kDecodeLaunchRows;
    const void* xr = static_cast<const uint16_t*>(x) + r0 * IC;
    void* orow = static_cast<uint16_t*>(out) + r0 * ldo;
    DecPlan pl;
    const bool i8_inblock = int8 && rows <= 4;
    if (!plan_decode(rows, IC, n, in, &pl, int8 && !i8_inblock))
      return fail(EXL3_EUNSUPPORTED, "%s: no decode-phase plan", who);
    if (i8_inblock) {
      int done = -1;
      for (int i = 0; i < n; ++i) {
        char* region = ws + L.xh_off + L.xh_bytes * size_t(slot[i]);
        float* part = reinterpret_cast<float*>(region + L.part_off);
        if (slot[i] > done) {
          if (L.xh_bytes < L.part_off + size_t(rows) * size_t(IC / 128) * 4)
            return fail(EXL3_EWORKSPACE, "%s: workspace has no 8-bit region", who);
          if (int rc = launch_status(launch_prepass_amax(xr, in[i].s_in, in[i].rin, part, rows, IC, stream), who))
            return rc;
          done = slot[i];
        }
        in[i].part = part;
      }
    }
    if (pl.pre) {
      int done = -1;
      for (int i = 0; i < n; ++i) {
        char* region = ws + L.xh_off + L.xh_bytes * size_t(slot[i]);
        float* scale = int8 ? reinterpret_cast<float*>(region + L.scale_off) : nullptr;
        if (slot[i] > done) {
          const size_t codes = size_t((rows + kDecodeMaxRows - 1) / kDecodeMaxRows * kDecodeMaxRows) * size_t(IC) * 2;
          if (L.xh_bytes < codes || (int8 && (L.scale_off < codes || L.part_off < L.scale_off + size_t(rows) * 4 ||
                                              L.xh_bytes < L.part_off + size_t(rows) * size_t(IC / 128) * 4)))
            return fail(EXL3_EWORKSPACE, "%s: workspace has no pre-rotation region", who);
          hipError_t e =
              int8 ? launch_prepass_i8(xr, in[i].s_in, in[i].rin, region, scale, rows, IC, true, stream, true,
                                       reinterpret_cast<float*>(region + L.part_off), false)
              : gu ? launch_prepass_silu_f16(static_cast<const uint16_t*>(gu) + r0 * 2 * IC, in[i].s_in, in[i].rin,
                                             region, rows, IC, stream)
                   : launch_prepass_f16(xr, in[i].s_in, in[i].rin, region, rows, IC, true, stream, kDecodeMaxRows);
          if (int rc = launch_status(e, who)) return rc;
          done = slot[i];
        }
        in[i].xf = region;
        in[i].sc = scale;
      }
    }
    if (gu && !pl.pre) {   // the folded activation in the in-block pre-pass (down is one shard)
      if (n != 1 || pl.kset < 0) return fail(EXL3_EUNSUPPORTED, "%s: folded activation needs one shard", who);
      hipError_t e = launch_decode(pl, static_cast<const uint16_t*>(gu) + r0 * 2 * IC, rows, IC, n, in, orow, ldo,
                                   reinterpret_cast<float*>(ws + L.slab_off), reinterpret_cast<int*>(ws), stream, true);
      if (int rc = launch_status(e, who)) return rc;
    } else if (pl.kset >= 0) {
      hipError_t e = launch_decode(pl, xr, rows, IC, n, in, orow, ldo, reinterpret_cast<float*>(ws + L.slab_off),
                                   reinterpret_cast<int*>(ws), stream, false, i8_inblock);
      if (int rc = launch_status(e, who)) return rc;
    } else {
      for (int i = 0; i < n; ++i) {
        DecPlan p1;
        if (!plan_decode(rows, IC, 1, in + i, &p1, int8 && !i8_inblock))
          return fail(EXL3_EUNSUPPORTED, "%s: no decode-phase plan", who);
        hipError_t e = launch_decode(p1, xr, rows, IC, 1, in + i, orow, ldo,
                                     reinterpret_cast<float*>(ws + L.slab_off), reinterpret_cast<int*>(ws), stream,
                                     false, i8_inblock);
        if (int rc = launch_status(e, who)) return rc;
      }
    }
  }
  return EXL3_OK;
}

// The prefill-phase path: one pre-pass per distinct (s_in, rin), then one GEMM per shard.  On the 8-bit
// path the pre-pass writes the integer codes (as fp16 numbers, exact) and the row scales, and the GEMM
// applies the row scale in its epilogue.
// gu (optional, 16-bit path only): as for run_decode.
int run_gemm(const char* who, void* out, int64_t ldo, const void* x, int64_t M, int64_t IC, int n, const DecShardIn* in,
             char* ws, const Layout& L, unsigned flags, hipStream_t stream, const void* gu = nullptr) {
  const bool int8 = (flags & EXL3_ACT_INT8) != 0;
  int slot[kMaxShards];
  distinct_inputs(n, in, slot);
  int done = -1;
  for (int i = 0; i < n; ++i) {
    char* region = ws + L.xh_off + L.xh_bytes * size_t(slot[i]);
    float* scale = int8 ? reinterpret_cast<float*>(region + L.scale_off) : nullptr;
    if (slot[i] > done) {
      hipError_t e = int8 ? launch_prepass_i8(x, in[i].s_in, in[i].rin, region, scale, M, IC, true, stream, true,
                                              reinterpret_cast<float*>(region + L.part_off), true)
                     : gu ? launch_prepass_silu_f16(gu, in[i].s_in, in[i].rin, region, M, IC, stream, true)
                          : launch_prepass_f16(x, in[i].s_in, in[i].rin, region, M, IC, true, stream, 0, true);
      if (int rc = launch_status(e, who)) return rc;
      done = slot[i];
    }
    const GemmSplit sp = (flags & kNoSplitFlags) ? GemmSplit{1, int(IC / 64)} : gemm_split(M, IC, in[i].OC);
    hipError_t e = launch_gemm(region, in[i].code, in[i].K, in[i].rout, in[i].s_out, out, ldo, in[i].col0, M, IC,
                               in[i].OC, stream, scale, sp, reinterpret_cast<float*>(ws + L.slab_off));
    if (int rc = launch_status(e, who)) return rc;
  }
  return EXL3_OK;
}

DecShardIn shard_in(const int16_t* code, int64_t OC, int K, int64_t col0, const void* s_in, const void* rin,
                    const void* rout, const void* s_out) {
  DecShardIn d;
  d.code = code;
  d.OC = OC;
  d.K = K;
  d.col0 = col0;
  d.s_in = s_in;
  d.rin = rin;
  d.rout = rout;
  d.s_out = s_out;
  return d;
}


// Workspace of the MoE bank forward: the route tables, then the per-pair rotated activations of w1 and
// w3, w2's rotated operand and the fp32 expert outputs.  The counter area at the head is kept for
// uniformity with the linear calls (unused here).
struct MoeLayout {
  size_t offs, pslot, rows, chunks, n_chunks, xh13, ah, o, total;
};

void moe_layout(int E, int H, int I, int64_t T, int topk, MoeLayout* L) {
  const size_t P = size_t(T) * size_t(topk);
  size_t at = align_up(kCounterBytes);
  auto take = [&](size_t bytes) {
    const size_t r = at;
    at += align_up(bytes ? bytes : 1);
    return r;
  };
  L->offs = take(size_t(E + 1) * 4);
  L->pslot = take(P * 4);
  L->rows = take(P * 4);
  L->chunks = take(size_t(moe_max_chunks(int64_t(P), E)) * 16);
  L->n_chunks = take(16);
  L->xh13 = take(2 * P * size_t(moe_row_pitch(H)) * 2);
  L->ah = take(P * size_t(moe_row_pitch(I)) * 2);
  L->o = take(P * size_t(H) * 4);
  L->total = at;
}

int check_bank(const exl3_bank* b) {
  if (!b) return fail(EXL3_EINVAL, "bank: null");
  if (b->E < 1 || b->E > kMoeMaxExperts) return fail(EXL3_EINVAL, "bank.E: %d is outside 1..%d", b->E, kMoeMaxExperts);
  if (b->H <= 0 || b->H % 128 || b->H > (1 << 16))
    return fail(EXL3_EINVAL, "bank.H: %d is not a positive multiple of 128 (at most 65536)", b->H);
  if (b->I <= 0 || b->I % 128 || b->I > (1 << 16))
    return fail(EXL3_EINVAL, "bank.I: %d is not a positive multiple of 128 (at most 65536)", b->I);
  if (b->n_groups < 1 || b->n_groups > kMoeMaxGroups)
    return fail(EXL3_EINVAL, "bank.n_groups: %d is outside 1..%d", b->n_groups, kMoeMaxGroups);
  if (!b->groups) return fail(EXL3_EINVAL, "bank.groups: null");
  int lo = 0;
  for (int g = 0; g < b->n_groups; ++g) {
    const exl3_group& G = b->groups[g];
    if (G.lo != lo || G.hi <= G.lo)
      return fail(EXL3_EINVAL, "bank.groups[%d]: [%d, %d) does not continue the slot ranges at %d", g, G.lo, G.hi, lo);
    if (G.k_gu < 1 || G.k_gu > 8 || G.k_d < 1 || G.k_d > 8)
      return fail(EXL3_EINVAL, "bank.groups[%d]: k_gu %d / k_d %d outside 1..8", g, G.k_gu, G.k_d);
    lo = G.hi;
  }
  if (lo != b->E) return fail(EXL3_EINVAL, "bank.groups: cover slots [0, %d), not [0, E=%d)", lo, b->E);
  if (!b->w13 || !b->w2 || !aligned(b->w13, 16) || !aligned(b->w2, 16))
    return fail(EXL3_EINVAL, "bank.w13/w2: null or not 16-byte aligned");
  if (!b->w13_suh || !b->w13_svh || !b->w2_suh || !b->w2_svh)
    return fail(EXL3_EINVAL, "bank.w13_suh/w13_svh/w2_suh/w2_svh: null");
  if (!aligned(b->w13_suh, 16)) return fail(EXL3_EINVAL, "bank.w13_suh: not 16-byte aligned");
  if (!aligned(b->w13_svh, 2) || !aligned(b->w2_suh, 2) || !aligned(b->w2_svh, 2))
    return fail(EXL3_EINVAL, "bank.w13_svh/w2_suh/w2_svh: not 2-byte aligned");
  if (!b->off_w1 || !b->off_w3 || !b->off_w2 || !aligned(b->off_w1, 8) || !aligned(b->off_w3, 8) ||
      !aligned(b->off_w2, 8))
    return fail(EXL3_EINVAL, "bank.off_w1/off_w3/off_w2: null or not 8-byte aligned");
  if (!b->perm || !aligned(b->perm, 4)) return fail(EXL3_EINVAL, "bank.perm: null or not 4-byte aligned");
  if (int64_t(b->H) * b->I >= (int64_t(1) << 31))
    return fail(EXL3_EUNSUPPORTED, "bank: H x I = %lld x %lld exceeds 2 GiB of trellis words per matrix",
                (long long)b->H, (long long)b->I);
  return EXL3_OK;
}

// Widest shard of a call: the GEMM runs one shard at a time, so its occupancy follows each shard's OC.
int64_t max_oc(int n, const DecShardIn* in) {
  int64_t m = 0;
  for (int i = 0; i < n; ++i) m = in[i].OC > m ? in[i].OC : m;
  return m;
}

// Workspace of either path for these shards (host descriptors; only OC, K and the s_in/rin pointers are read).
bool workspace_layout(int64_t M, int64_t IC, int n, const DecShardIn* in, unsigned flags, Layout* L) {
  if (use_decode_path(M, flags, max_oc(n, in))) {
    const bool int8 = (flags & EXL3_ACT_INT8) != 0;
    size_t slab = 0;
    if (!decode_slab_bytes(M, IC, n, in, &slab, int8)) return false;
    int slot[kMaxShards];
    const bool pre = int8 || first_chunk(M) >= kPreRotateRows || last_chunk(M) >= kPreRotateRows;
    *L = layout_for(slab, pre_rows(M), IC, pre ? distinct_inputs(n, in, slot) : 0, int8, kDecodeMaxRows);
  } else {
    size_t slab = 0;                                      // shards run one after another: the largest split
    if (!(flags & kNoSplitFlags))
      for (int i = 0; i < n; ++i) {
        const size_t b = gemm_slab_bytes(M, in[i].OC, gemm_split(M, IC, in[i].OC));
        slab = b > slab ? b : slab;
      }
    int slot[kMaxShards];
    *L = layout_for(slab, M, IC, distinct_inputs(n, in, slot), (flags & EXL3_ACT_INT8) != 0);
  }
  return true;
}

}  // namespace

namespace exl3 {
// int8 embedding gather (k_embed.hip): out bf16 [T, H] = table[ids] * scale[ids]; zero rows for ids
// outside [0, V).
hipError_t launch_embed_int8(void* out, const int8_t* table, const void* scale, int64_t V, int64_t H,
                             const int32_t* ids, int64_t T, hipStream_t stream);
// the int8 table as the output head (k_embed.hip): logits bf16 [M, V] (row stride ldo) =
// x [M, H] . bf16(table * scale)^T.
hipError_t launch_lm_head_int8(void* out, int64_t ldo, const void* x, int64_t M, const int8_t* table,
                               const void* scale, int64_t V, int64_t H, hipStream_t stream);
// dense MLP activation (k_mlp.hip): h bf16 [M, I] = bf16(silu(gu[:, :I]) * gu[:, I:]) of a bf16 [M, 2I] input.
hipError_t launch_silu_mul(void* h, const void* gu, int64_t M, int64_t I, hipStream_t stream);
}  // namespace exl3

extern "C" {

const char* exl3_last_error(void) { return g_error.c_str(); }

int exl3_version(void) { return 100; }

int64_t exl3_gemv_max_rows(int64_t OC) { return gemv_max_rows(OC); }

int exl3_gemm_splits(int64_t M, int64_t IC, int64_t OC) {
  if (M <= 0 || IC <= 0 || OC <= 0 || IC % 128 || OC % 128) return 1;
  return gemm_split(M, IC, OC).splits;
}

int exl3_gemm_tail_splits(int64_t M, int64_t IC, int64_t OC) {
  if (M <= 0 || IC <= 0 || OC <= 0 || IC % 128 || OC % 128) return 1;
  const GemmSplit sp = gemm_split(M, IC, OC);
  return sp.splits > 1 ? 1 : sp.tail_splits;
}

size_t exl3_linear_workspace_bytes(int64_t M, int64_t IC, int64_t OC, unsigned flags) {
  if (M <= 0 || IC <= 0 || OC <= 0 || IC % 128 || OC % 128) return align_up(kCounterBytes);
  const DecShardIn in = shard_in(nullptr, OC, 2, 0, nullptr, nullptr, nullptr, nullptr);
  Layout L;
  if (!workspace_layout(M, IC, 1, &in, flags, &L)) return align_up(kCounterBytes);
  return L.total;
}

}  // extern "C"

namespace {
int linear_into_impl(void* out, int64_t ldo, int64_t col0, const void* x, int64_t M, int64_t IC, const int16_t* code,
                     int64_t OC, int K, const void* s_in, const void* rin, const void* rout, const void* s_out,
                     unsigned flags, void* ws, size_t ws_bytes, void* stream, const void* gu) {
  if (int rc = check_flags(flags)) return rc;
  if (int rc = check_dims(M, IC)) return rc;
  if (int rc = check_shard("", IC, code, OC, K, col0, ldo, s_in, rin, rout, s_out)) return rc;
  if (M == 0) return ok();
  if (!out || !aligned(out, 16)) return fail(EXL3_EINVAL, "out: null or not 16-byte aligned");
  if (!x || !aligned(x, 16)) return fail(EXL3_EINVAL, "x: null or not 16-byte aligned");
  const DecShardIn in = shard_in(code, OC, K, col0, s_in, rin, rout, s_out);
  Layout L;
  if (!workspace_layout(M, IC, 1, &in, flags, &L)) return fail(EXL3_EUNSUPPORTED, "exl3_linear_into: no plan");
  if (int rc = check_workspace(L, ws, ws_bytes)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rc = use_decode_path(M, flags, OC)
                     ? run_decode("exl3_linear_into", out, ldo, x, M, IC, 1, &in, static_cast<char*>(ws), L, st, gu,
                                  (flags & EXL3_ACT_INT8) != 0)
                     : run_gemm("exl3_linear_into", out, ldo, x, M, IC, 1, &in, static_cast<char*>(ws), L, flags, st, gu);
  if (rc) return rc;
  return ok();
}
}  // namespace

extern "C" {

int exl3_linear_into(void* out, int64_t ldo, int64_t col0, const void* x, int64_t M, int64_t IC,
                     const int16_t* code, int64_t OC, int K, const void* s_in, const void* rin, const void* rout,
                     const void* s_out, unsigned flags, void* ws, size_t ws_bytes, void* stream) {
  return linear_into_impl(out, ldo, col0, x, M, IC, code, OC, K, s_in, rin, rout, s_out, flags, ws, ws_bytes, stream,
                          nullptr);
}

size_t exl3_linear_multi_workspace_bytes(int64_t M, int64_t IC, int n_shards, const exl3_shard* shards,
                                         unsigned flags) {
  if (M <= 0 || IC <= 0 || IC % 128 || n_shards <= 0 || n_shards > kMaxShards || !shards) return align_up(kCounterBytes);
  DecShardIn in[kMaxShards];
  for (int i = 0; i < n_shards; ++i) {
    if (shards[i].OC <= 0 || shards[i].OC % 128) return align_up(kCounterBytes);
    in[i] = shard_in(nullptr, shards[i].OC, shards[i].K, 0, shards[i].s_in, shards[i].rin, nullptr, nullptr);
  }
  Layout L;
  if (!workspace_layout(M, IC, n_shards, in, flags, &L)) return align_up(kCounterBytes);
  return L.total;
}

int exl3_linear_multi_into(void* out, int64_t ldo, const void* x, int64_t M, int64_t IC, int n_shards,
                           const exl3_shard* shards, unsigned flags, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = check_flags(flags)) return rc;
  if (int rc = check_dims(M, IC)) return rc;
  if (n_shards < 1 || n_shards > kMaxShards) return fail(EXL3_EINVAL, "n_shards: %d is outside 1..16", n_shards);
  if (!shards) return fail(EXL3_EINVAL, "shards: null");
  DecShardIn in[kMaxShards];
  for (int i = 0; i < n_shards; ++i) {
    const exl3_shard& s = shards[i];
    char who[32];
    snprintf(who, sizeof who, "shards[%d].", i);
    if (int rc = check_shard(who, IC, s.code, s.OC, s.K, s.col0, ldo, s.s_in, s.rin, s.rout, s.s_out)) return rc;
    in[i] = shard_in(s.code, s.OC, s.K, s.col0, s.s_in, s.rin, s.rout, s.s_out);
  }
  if (M == 0) return ok();
  if (!out || !aligned(out, 16)) return fail(EXL3_EINVAL, "out: null or not 16-byte aligned");
  if (!x || !aligned(x, 16)) return fail(EXL3_EINVAL, "x: null or not 16-byte aligned");
  Layout L;
  if (!workspace_layout(M, IC, n_shards, in, flags, &L)) return fail(EXL3_EUNSUPPORTED, "exl3_linear_multi_into: no plan");
  if (int rc = check_workspace(L, ws, ws_bytes)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rc = use_decode_path(M, flags, max_oc(n_shards, in))
                     ? run_decode("exl3_linear_multi_into", out, ldo, x, M, IC, n_shards, in, static_cast<char*>(ws), L, st,
                                  nullptr, (flags & EXL3_ACT_INT8) != 0)
                     : run_gemm("exl3_linear_multi_into", out, ldo, x, M, IC, n_shards, in, static_cast<char*>(ws), L, flags,
                                st);
  if (rc) return rc;
  return ok();
}

size_t exl3_moe_workspace_bytes(const exl3_bank* bank, int64_t T, int topk, unsigned flags) {
  (void)flags;
  MoeLayout L;
  if (!bank || T < 0 || topk < 1 || bank->E < 1 || bank->H <= 0 || bank->I <= 0) return align_up(kCounterBytes);
  moe_layout(bank->E, bank->H, bank->I, T, topk, &L);
  return L.total;
}

int exl3_moe_bank_forward(void* out, const void* x, int64_t T, const int32_t* topk_ids, const float* topk_w, int topk,
                          const exl3_bank* bank, unsigned flags, void* ws, size_t ws_bytes, void* stream) {
  if (flags & EXL3_ACT_INT8) return fail(EXL3_EUNSUPPORTED, "flags: EXL3_ACT_INT8 is not available for the MoE bank");
  if (flags & ~unsigned(EXL3_FORCE_GEMV | EXL3_FORCE_MFMA))
    return fail(EXL3_EINVAL, "flags: 0x%x has no meaning for the MoE bank", flags);
  if ((flags & EXL3_FORCE_GEMV) && (flags & EXL3_FORCE_MFMA))
    return fail(EXL3_EINVAL, "flags: EXL3_FORCE_GEMV and EXL3_FORCE_MFMA are exclusive");
  if (int rc = check_bank(bank)) return rc;
  if (topk < 1 || topk > bank->E) return fail(EXL3_EINVAL, "topk: %d is outside 1..E (%d)", topk, bank->E);
  if (T < 0) return fail(EXL3_EINVAL, "T: %lld is negative", (long long)T);
  if (T * topk > (int64_t(1) << 24)) return fail(EXL3_EINVAL, "T: %lld x topk %d exceeds 2^24 pairs", (long long)T, topk);
  if (T == 0) return ok();
  if (!out || !aligned(out, 16)) return fail(EXL3_EINVAL, "out: null or not 16-byte aligned");
  if (!x || !aligned(x, 16)) return fail(EXL3_EINVAL, "x: null or not 16-byte aligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(EXL3_EINVAL, "topk_ids: null or not 4-byte aligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(EXL3_EINVAL, "topk_w: null or not 4-byte aligned");
  MoeLayout L;
  moe_layout(bank->E, bank->H, bank->I, T, topk, &L);
  if (!ws) return fail(EXL3_EWORKSPACE, "ws: null (need %zu bytes)", L.total);
  if (!aligned(ws, kAlign)) return fail(EXL3_EINVAL, "ws: not %zu-byte aligned", kAlign);
  if (ws_bytes < L.total) return fail(EXL3_EWORKSPACE, "ws_bytes: %zu < required %zu", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  MoeLaunch m;
  m.x = x;
  m.ids = topk_ids;
  m.wts = topk_w;
  m.perm = bank->perm;
  m.w13 = bank->w13;
  m.w2 = bank->w2;
  m.w13_suh = bank->w13_suh;
  m.w13_svh = bank->w13_svh;
  m.w2_suh = bank->w2_suh;
  m.w2_svh = bank->w2_svh;
  m.off_w1 = bank->off_w1;
  m.off_w3 = bank->off_w3;
  m.off_w2 = bank->off_w2;
  m.out = out;
  m.offs = reinterpret_cast<int32_t*>(w + L.offs);
  m.pslot = reinterpret_cast<int32_t*>(w + L.pslot);
  m.rows = reinterpret_cast<int32_t*>(w + L.rows);
  m.chunks = reinterpret_cast<int32_t*>(w + L.chunks);
  m.n_chunks = reinterpret_cast<int32_t*>(w + L.n_chunks);
  m.xh13 = w + L.xh13;
  m.ah = w + L.ah;
  m.o = reinterpret_cast<float*>(w + L.o);
  m.T = T;
  m.topk = topk;
  m.E = bank->E;
  m.H = bank->H;
  m.I = bank->I;
  m.n_groups = bank->n_groups;
  for (int g = 0; g < kMoeMaxGroups; ++g) {
    m.g_hi[g] = g < bank->n_groups ? bank->groups[g].hi : 0;
    m.g_k[g] = g < bank->n_groups ? (bank->groups[g].k_gu | (bank->groups[g].k_d << 8)) : 0;
  }
  m.plan = (flags & EXL3_FORCE_GEMV) ? 1 : (flags & EXL3_FORCE_MFMA) ? 2 : 0;
  if (m.plan == 2 && !moe_prefill_plan(T * topk, bank->E, bank->H, bank->I, 2))
    return fail(EXL3_EUNSUPPORTED, "flags: EXL3_FORCE_MFMA: T * topk x max(H, I) fp16 exceeds 2 GiB for the prefill plan");
  if (int rc = launch_status(launch_moe(m, static_cast<hipStream_t>(stream)), "exl3_moe_bank_forward")) return rc;
  return ok();
}

int exl3_embed_int8(void* out, const int8_t* table, const void* scale, int64_t V, int64_t H, const int32_t* ids,
                    int64_t T, void* stream) {
  if (T < 0) return fail(EXL3_EINVAL, "T: %lld is negative", (long long)T);
  if (V < 1) return fail(EXL3_EINVAL, "V: %lld rows", (long long)V);
  if (H < 16 || H % 16) return fail(EXL3_EINVAL, "H: %lld is not a positive multiple of 16", (long long)H);
  if (T == 0) return ok();
  if (!out || !table || !scale || !ids) return fail(EXL3_EINVAL, "out/table/scale/ids: null");
  if (!aligned(out, 16) || !aligned(table, 16)) return fail(EXL3_EINVAL, "out/table: not 16-byte aligned");
  if (!aligned(scale, 2) || !aligned(ids, 4)) return fail(EXL3_EINVAL, "scale/ids: not 2-/4-byte aligned");
  if (int rc = launch_status(launch_embed_int8(out, table, scale, V, H, ids, T, static_cast<hipStream_t>(stream)),
                             "exl3_embed_int8"))
    return rc;
  return ok();
}

int exl3_lm_head_int8(void* out, int64_t ldo, const void* x, int64_t M, const int8_t* table, const void* scale,
                      int64_t V, int64_t H, void* stream) {
  if (M < 0) return fail(EXL3_EINVAL, "M: %lld is negative", (long long)M);
  if (V < 1) return fail(EXL3_EINVAL, "V: %lld rows", (long long)V);
  if (H < 64 || H % 64) return fail(EXL3_EINVAL, "H: %lld is not a positive multiple of 64", (long long)H);
  if (ldo < V) return fail(EXL3_EINVAL, "ldo: %lld is below V", (long long)ldo);
  if (M == 0) return ok();
  if (!out || !x || !table || !scale) return fail(EXL3_EINVAL, "out/x/table/scale: null");
  if (!aligned(x, 16) || !aligned(table, 16)) return fail(EXL3_EINVAL, "x/table: not 16-byte aligned");
  if (!aligned(out, 2) || !aligned(scale, 2)) return fail(EXL3_EINVAL, "out/scale: not 2-byte aligned");
  if (int rc = launch_status(launch_lm_head_int8(out, ldo, x, M, table, scale, V, H, static_cast<hipStream_t>(stream)),
                             "exl3_lm_head_int8"))
    return rc;
  return ok();
}

// Dense MLP block: the workspace holds, in order, the projections' own workspace (its counter area first, so
// zeroing the whole buffer once zeroes it), the gate_up output bf16 [M, 2I] and the activation bf16 [M, I].
namespace {
struct MlpLayout {
  size_t inner, gu_off, h_off, total;
};

bool mlp_layout(int64_t M, int64_t H, int64_t I, const exl3_shard* gate, const exl3_shard* up, unsigned flags,
                MlpLayout* L) {
  exl3_shard gu[2] = {*gate, *up};
  gu[0].col0 = 0;
  gu[1].col0 = I;
  const size_t a = exl3_linear_multi_workspace_bytes(M, H, 2, gu, flags);
  const size_t b = exl3_linear_workspace_bytes(M, I, H, flags);
  L->inner = align_up(a > b ? a : b);
  L->gu_off = L->inner;
  L->h_off = L->gu_off + align_up(size_t(M) * 2 * I * 2);
  L->total = L->h_off + align_up(size_t(M) * I * 2);
  return true;
}

int check_mlp(int64_t M, int64_t H, int64_t I, const exl3_shard* gate, const exl3_shard* up, const exl3_shard* down) {
  if (M < 0) return fail(EXL3_EINVAL, "M: %lld is negative", (long long)M);
  if (H < 128 || H % 128) return fail(EXL3_EINVAL, "H: %lld is not a positive multiple of 128", (long long)H);
  if (I < 128 || I % 128) return fail(EXL3_EINVAL, "I: %lld is not a positive multiple of 128", (long long)I);
  if (!gate || !up || !down) return fail(EXL3_EINVAL, "gate/up/down: null");
  if (gate->OC != I || up->OC != I) return fail(EXL3_EINVAL, "gate/up: OC must equal I");
  if (down->OC != H) return fail(EXL3_EINVAL, "down: OC must equal H");
  return 0;
}
}  // namespace

size_t exl3_mlp_workspace_bytes(int64_t M, int64_t H, int64_t I, const exl3_shard* gate, const exl3_shard* up,
                                unsigned flags) {
  if (M <= 0 || !gate || !up || H < 128 || H % 128 || I < 128 || I % 128) return align_up(kCounterBytes);
  MlpLayout L;
  mlp_layout(M, H, I, gate, up, flags, &L);
  return L.total;
}

int exl3_mlp_forward(void* out, const void* x, int64_t M, int64_t H, int64_t I, const exl3_shard* gate,
                     const exl3_shard* up, const exl3_shard* down, unsigned flags, void* ws, size_t ws_bytes,
                     void* stream) {
  if (int rc = check_flags(flags)) return rc;
  if (int rc = check_mlp(M, H, I, gate, up, down)) return rc;
  if (M == 0) return ok();
  if (!ws) return fail(EXL3_EWORKSPACE, "ws: null");
  if (!aligned(ws, kAlign)) return fail(EXL3_EINVAL, "ws: not %zu-byte aligned", kAlign);
  MlpLayout L;
  mlp_layout(M, H, I, gate, up, flags, &L);
  if (ws_bytes < L.total)
    return fail(EXL3_EWORKSPACE, "ws_bytes: %zu < %zu (exl3_mlp_workspace_bytes)", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  exl3_shard gu[2] = {*gate, *up};
  gu[0].col0 = 0;
  gu[1].col0 = I;
  if (int rc = exl3_linear_multi_into(w + L.gu_off, 2 * I, x, M, H, 2, gu, flags, w, L.inner, stream)) return rc;
  // on the 16-bit path down's activation pre-pass (the rotation launch, or the decode kernel's in-block
  // pre-pass for 1..4 rows) forms h itself; only the 8-bit pre-pass reads h from memory
  const bool int8 = (flags & EXL3_ACT_INT8) != 0;
  const bool fold = !int8;
  const bool need_h = int8;
  if (need_h) {
    if (int rc = launch_status(launch_silu_mul(w + L.h_off, w + L.gu_off, M, I, static_cast<hipStream_t>(stream)),
                               "exl3_mlp_forward"))
      return rc;
  }
  if (int rc = linear_into_impl(out, H, 0, w + L.h_off, M, I, down->code, H, down->K, down->s_in, down->rin,
                                down->rout, down->s_out, flags, w, L.inner, stream, fold ? w + L.gu_off : nullptr))
    return rc;
  return ok();
}

int exl3_silu_mul(void* h, const void* gu, int64_t M, int64_t I, void* stream) {
  if (M < 0) return fail(EXL3_EINVAL, "M: %lld is negative", (long long)M);
  if (I < 8 || I % 8) return fail(EXL3_EINVAL, "I: %lld is not a positive multiple of 8", (long long)I);
  if (M == 0) return ok();
  if (!h || !gu || !aligned(h, 16) || !aligned(gu, 16)) return fail(EXL3_EINVAL, "h/gu: null or not 16-byte aligned");
  if (int rc = launch_status(launch_silu_mul(h, gu, M, I, static_cast<hipStream_t>(stream)), "exl3_silu_mul"))
    return rc;
  return ok();
}

int exl3_decode_tiles(void* w_out, const int16_t* code, int64_t IC, int64_t OC, int K, void* stream) {
  if (IC <= 0 || IC % 16 || OC <= 0 || OC % 16)
    return fail(EXL3_EINVAL, "IC/OC: %lld x %lld are not positive multiples of 16", (long long)IC, (long long)OC);
  if (K < 1 || K > 8) return fail(EXL3_EINVAL, "K: %d is outside 1..8", K);
  if (!w_out || !code) return fail(EXL3_EINVAL, "w_out/code: null");
  if (!aligned(code, 16)) return fail(EXL3_EINVAL, "code: not 16-byte aligned");
  if (!aligned(w_out, 2)) return fail(EXL3_EINVAL, "w_out: not 2-byte aligned");
  if (int rc = launch_status(launch_decode_tiles(w_out, code, IC, OC, K, static_cast<hipStream_t>(stream)),
                             "exl3_decode_tiles"))
    return rc;
  return ok();
}

int exl3_rotate_activations(void* q_out, float* scale_out, const void* x, int64_t M, int64_t IC, const void* s_in,
                            const void* rin, unsigned flags, void* stream) {
  if (flags & ~unsigned(EXL3_ACT_INT8)) return fail(EXL3_EINVAL, "flags: only EXL3_ACT_INT8 is meaningful here");
  if (int rc = check_dims(M, IC)) return rc;
  if (M == 0) return ok();
  if (!q_out || !x || !s_in || !rin) return fail(EXL3_EINVAL, "q_out/x/s_in/rin: null");
  if (!aligned(x, 16) || !aligned(q_out, 16)) return fail(EXL3_EINVAL, "x/q_out: not 16-byte aligned");
  if (!aligned(s_in, 4) || !aligned(rin, 4)) return fail(EXL3_EINVAL, "s_in/rin: not 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (flags & EXL3_ACT_INT8) {
    if (!scale_out) return fail(EXL3_EINVAL, "scale_out: null");
    e = launch_prepass_i8(x, s_in, rin, q_out, scale_out, M, IC, false, st);
  } else {
    e = launch_prepass_f16(x, s_in, rin, q_out, M, IC, false, st);
  }
  if (int rc = launch_status(e, "exl3_rotate_activations")) return rc;
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------------
// Allocation-free variant of exl3_linear_multi_into.  Its workspace is `scratch`, a file-scope device
// array of kStaticScratchBytes: every GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address (on the host it is only a stand-in): the
// first call on a device looks up that device's copy with hipGetSymbolAddress, with the device current,
// and keeps the address.  The split-K counters at the head of the workspace must start at zero; that
// first call clears them with a fill kernel on the caller's stream, and every kernel leaves them at zero
// again when it ends.  Every call on a device shares its copy, so calls that may overlap on one device
// (different streams, different threads without ordering) race.
// ---------------------------------------------------------------------------------------------------
namespace {

constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < n) p[i] = 0u;
}

// This device's copy of `scratch`, set up on the first call made with the device current.
int static_scratch(void** ptr, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(EXL3_ELAUNCH, "static scratch: no usable current device (%d)", dev);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(EXL3_ELAUNCH, "static scratch: hipGetSymbolAddress failed on device %d: %s", dev, hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words_kernel, dim3((kCounterSlots + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), kCounterSlots);
    if (int rc = launch_status(hipGetLastError(), "static scratch: clearing the counters")) return rc;
    g_static_ptr[dev] = p;
  }
  *ptr = g_static_ptr[dev];
  return EXL3_OK;
}

}  // namespace

extern "C" {

int exl3_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int variant, void* stream) {
  if (!src || !sink) return fail(EXL3_EINVAL, "src/sink: null");
  if (!aligned(src, 16) || bytes % 16) return fail(EXL3_EINVAL, "src/bytes: not 16-byte aligned");
  if (blocks < 1 || blocks > (1 << 20)) return fail(EXL3_EINVAL, "blocks: %d is outside 1..2^20", blocks);
  if (variant < 0 || variant > 2) return fail(EXL3_EINVAL, "variant: %d is outside 0..2", variant);
  if (int rc = launch_status(launch_probe_read(src, bytes, sink, blocks, variant, static_cast<hipStream_t>(stream)),
                             "exl3_probe_read"))
    return rc;
  return ok();
}

int exl3_probe_mfma(float* sink, int kind, int iters, int blocks, void* stream) {
  if (!sink) return fail(EXL3_EINVAL, "sink: null");
  if (kind < 0 || kind > 3) return fail(EXL3_EINVAL, "kind: %d is outside 0..3", kind);
  if (iters < 1) return fail(EXL3_EINVAL, "iters: %d < 1", iters);
  if (blocks < 1 || blocks > (1 << 20)) return fail(EXL3_EINVAL, "blocks: %d is outside 1..2^20", blocks);
  if (int rc = launch_status(launch_probe_mfma(sink, kind, iters, blocks, static_cast<hipStream_t>(stream)),
                             "exl3_probe_mfma"))
    return rc;
  return ok();
}

size_t exl3_static_scratch_bytes(void) { return kStaticScratchBytes; }

int exl3_linear_multi_into_static(void* out, int64_t ldo, const void* x, int64_t M, int64_t IC, int n_shards,
                                  const exl3_shard* shards, unsigned flags, void* stream) {
  const size_t need = exl3_linear_multi_workspace_bytes(M, IC, n_shards, shards, flags);
  if (need > kStaticScratchBytes)
    return fail(EXL3_EWORKSPACE,
                "exl3_linear_multi_into_static: this call needs %zu bytes of scratch, the static scratch holds %zu; "
                "use exl3_linear_multi_into with a workspace", need, kStaticScratchBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (int rc = static_scratch(&ws, st)) return rc;
  return exl3_linear_multi_into(out, ldo, x, M, IC, n_shards, shards, flags, ws, kStaticScratchBytes, stream);
}

}  // extern "C"
