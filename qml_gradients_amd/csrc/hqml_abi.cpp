// C ABI of the hqml library: argument checks, workspace ownership, and the order
// of kernel launches for forward, backward and training steps.
//
// Backward gate fusion (hugo-pages summary, section 1.4 item 2): each backward
// pass reads the saved output of one fused forward pass and the adjoint state,
// re-derives the pass's input on chip with U^dagger while forming the gradient
// terms, and writes the propagated adjoint state.  Gradient checkpointing
// (section 2.3): with ckpt_block = b, only one state every b layers is kept and a
// block's forward passes are recomputed just before its backward passes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/hqml.h"
#include "hqml_internal.hpp"
#include "hqml_plan.hpp"

#include "hqml_host.hpp"

using namespace hqml;

struct hqml_ctx {
    hqml_config cfg{};
    Plan plan;
    Workspace ws;
    hipStream_t stream = nullptr;
    // Second stream (default priority, non-blocking): in a training step the batch is
    // split into chunks; chunk k+1's forward sweep runs there while chunk k's adjoint
    // sweep runs on 'stream' (the forward is memory-bound, the adjoint ALU-bound).
    hipStream_t aux = nullptr;
    hipEvent_t ev_start = nullptr;
    hipEvent_t ev_fwd[8] = {};
    int chunks = 0;              // 0: automatic
    std::vector<void *> allocs;
    // device buffers
    int r64 = 0;                 // compute type: 0 float, 1 double
    size_t rb = 4;               // bytes of the compute type
    char *saved = nullptr;       // saved states (n_saved buffers of max_batch samples)
    void *lam = nullptr;         // arrays below in the compute type
    void *lam_alt = nullptr;     // CNOT plan: second lambda buffer for the passes that scatter it
    // The two lambda allocations.  'lam' / 'lam_alt' swap roles after every pass that
    // scatters lambda; each backward sweep starts from lam_buf[0], where the
    // observable pass writes its seed.
    void *lam_buf[2] = {nullptr, nullptr};
    char *part = nullptr;
    void *e_part = nullptr;
    double *S = nullptr;
    double *zyz = nullptr;
    unsigned char *frame = nullptr;
    void *rot_tf = nullptr;
    void *dw = nullptr;
    double *H = nullptr;
    void *init_u = nullptr;
    ViewDev *views = nullptr;
    ViewDevH *hviews = nullptr;  // half-tile views (general adjoint passes on half tiles)
    bool half = false;           // tile plan whose views all have half views
    int stat_mul = 1;            // statistics partials per full tile: 2 with half tiles
    int2 *statmap = nullptr;
    double *dlde = nullptr;
    double *e_work = nullptr;
    double *part2 = nullptr;    // first-stage statistics sums (samples with many tiles)
    double *epart2 = nullptr;   // first-stage <O> sums
    float *loss_tmp = nullptr;
    uint32_t obs = 1;            // observable: Z part of the Pauli string
    uint32_t obs_x = 0;          // observable: X part (Y where both); nonzero adds an observable pass
    bool obs_neg = false;        // CNOT-chain plan: the conjugated string carries a sign -1
    // gate-by-gate comparator
    bool gbg = false;
    float *gbg_psi = nullptr;    // [B][2^n] complex fp32
    float *gbg_lam = nullptr;
    double *gbg_part = nullptr;  // [3nL][B][blocks] gradient block sums
    float *gbg_theta = nullptr;  // theta of the saved forward
    int gbg_blocks = 0;
    // saved-forward bookkeeping
    int saved_B = -1;
    // Checkpointed plans keep the last block's pass outputs in the block buffers, which
    // a backward sweep's recomputation of the other blocks overwrites: false once that
    // has happened, so a later backward on the same saved forward recomputes the block.
    bool tail_valid = false;
    std::string err;
    // caller arrays already found device-accessible and large enough, one slot per argument
    struct Checked {
        const void *p = nullptr;
        size_t bytes = 0;
        const void *base = nullptr;   // the allocation that held it
        size_t size = 0;
    };
    Checked checked[8];
    // instrumentation
    bool timing = false;
    struct Rec {
        int kind;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
    size_t pool_used = 0;
};

namespace {

thread_local std::string g_create_err;

int fail(hqml_ctx *c, int code, const std::string &msg)
{
    if (c) c->err = msg;
    else g_create_err = msg;
    return code;
}

int hip_fail(hqml_ctx *c, hipError_t e, const char *what)
{
    return fail(c, HQML_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Caller array argument `slot` (its index in the table above): see check_device_array.
// A pointer that passed is remembered per slot together with its allocation's base and
// size; a later call with the same pointer re-reads only the allocation range (a cheap
// host-side lookup), so a buffer freed and replaced by a different allocation at the
// same address is checked again in full.
int check_array(hqml_ctx *c, int slot, const void *p, size_t bytes, const char *name)
{
    hqml_ctx::Checked &k = c->checked[slot];
    if (p && p == k.p && bytes <= k.bytes) {
        void *b = nullptr;
        size_t sz = 0;
        if (hipMemGetAddressRange(&b, &sz, const_cast<void *>(p)) == hipSuccess && b == k.base && sz == k.size)
            return HQML_OK;
        (void)hipGetLastError();
        k = hqml_ctx::Checked{};
    }
    std::string err;
    const void *base = nullptr;
    size_t size = 0;
    const int rc = check_device_array(c->cfg.device, p, bytes, name, &err, &base, &size);
    if (rc != HQML_OK) return fail(c, rc, err);
    k.p = p;
    k.bytes = bytes;
    k.base = base;
    k.size = size;
    return HQML_OK;
}

size_t elem_bytes(const hqml_ctx *c)
{
    return c->cfg.storage == HQML_STORE_BF16 ? 4 : c->cfg.storage == HQML_STORE_FP64 ? 16 : 8;
}

hipEvent_t take_event(hqml_ctx *c)
{
    if (c->pool_used == c->pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        c->pool.push_back(e);
    }
    return c->pool[c->pool_used++];
}

template <class F>
int run_on(hqml_ctx *c, hipStream_t st, int kind, const char *what, F f)
{
    hipEvent_t a = nullptr, b = nullptr;
    if (c->timing) {
        a = take_event(c);
        b = take_event(c);
        if (a && b) (void)hipEventRecord(a, st);
    }
    hipError_t e = f();
    if (c->timing && a && b) {
        (void)hipEventRecord(b, st);
        c->recs.push_back({kind, a, b});
    }
    if (e != hipSuccess) return hip_fail(c, e, what);
    return HQML_OK;
}

template <class F>
int run(hqml_ctx *c, int kind, const char *what, F f)
{
    return run_on(c, c->stream, kind, what, f);
}

// A chunk of the batch: samples b0 .. b0+bc-1 of a batch of bs samples.
struct Span {
    int b0, bc, bs;
};

// Saved state buffer i (each holds max_batch samples).
void *saved_buf(hqml_ctx *c, int i)
{
    return c->saved + (size_t)i * c->ws.state_bytes;
}

// Where the output of forward pass p lives (same mapping in the forward sweep, the
// checkpoint recompute and the backward sweep).
void *pass_out(hqml_ctx *c, int p)
{
    const Plan &pl = c->plan;
    if (pl.c == 0) return saved_buf(c, p);
    const int k = p / pl.c, lo = k * pl.c;
    const int P = pl.n_fwd();
    const int hi = std::min(P, lo + pl.c);
    if (p == hi - 1 && k < pl.nblocks - 1) return saved_buf(c, pl.c + k);   // checkpoint k+1
    return saved_buf(c, p - lo);
}

TilePassArgs base_args(hqml_ctx *c)
{
    TilePassArgs a;
    std::memset(&a, 0, sizeof a);
    a.lam = c->lam;
    a.e_part = c->e_part;
    a.rot_tf = c->rot_tf;
    a.dw = c->dw;
    a.init_u = c->init_u;
    a.n = c->plan.n;
    a.L = c->plan.L;
    a.T = c->plan.T;
    a.obs = c->obs;
    a.obs_x = c->obs_x;
    a.stat_mul = c->stat_mul;
    return a;
}

int fwd_pass(hqml_ctx *c, hipStream_t st, Span sp, int p, int extra_flags)
{
    const PassPlan &pp = c->plan.fwd[p];
    TilePassArgs a = base_args(c);
    a.view = c->views + pp.view;
    a.psi_in = p == 0 ? nullptr : pass_out(c, p - 1);
    a.psi_out = pass_out(c, p);
    a.rotA = pp.rotA;
    a.diag = pp.diag;
    a.rotB = pp.rotB;
    a.flags = (pp.init ? PF_INIT : 0) | PF_STORE | extra_flags;
    if (c->plan.cnot) a.flags |= PF_CNOT | (pp.gather ? PF_GATHER : 0);
    a.sample0 = sp.b0;
    return run_on(c, st, HQML_K_FWD_PASS, "forward pass launch",
                  [&] { return launch_tile_fwd(a, sp.bc, c->cfg.storage, c->r64, st); });
}

// Backward pass k (forward pass index, or n_fwd + i for the i-th layer-0 stats-only pass).
int bwd_pass(hqml_ctx *c, hipStream_t st, Span sp, int k, int part_lo, char *part_base, int extra_flags)
{
    const Plan &pl = c->plan;
    const int P = pl.n_fwd();
    TilePassArgs a = base_args(c);
    a.stat_part = part_base + (size_t)(k - part_lo) * sp.bs * pl.T * c->stat_mul * kSlots * c->rb;
    a.sample0 = sp.b0;
    if (k >= P) {
        a.view = c->views + pl.stats_only[k - P];
        a.rotA = a.diag = a.rotB = -1;
        a.flags = PF_STATS_ONLY | PF_INIT;
        if (pl.cnot) {   // lambda is taken back through diag(p_0) first
            a.diag = 0;
            a.flags |= PF_CNOT;
        }
    } else if (pl.cnot && k == 0) {   // the product-state pass: its backward is layer-0 statistics
        a.view = c->views;
        a.rotA = a.rotB = -1;
        a.diag = 0;
        a.flags = PF_STATS_ONLY | PF_INIT | PF_CNOT | (extra_flags & PF_SEED);
    } else {
        const PassPlan &pp = pl.fwd[k];
        a.view = c->views + pp.view;
        a.rotA = pp.rotA;
        a.diag = pp.diag;
        a.rotB = pp.rotB;
        a.flags = (pp.init ? PF_INIT : 0) | extra_flags;
        if (pl.cnot) a.flags |= PF_CNOT | (pp.gather ? PF_GATHER : 0);
        if (extra_flags & PF_FUSED)
            a.psi_in = k == 0 ? nullptr : pass_out(c, k - 1);
        else
            a.psi_in = pass_out(c, k);
        // half tiles when the context has them: the general shape [rotA, D, rotB] of the CZ
        // chain, the CNOT chain's [rotA, diag(p_l)] and [diag(r_l), rotB] (on a saved output,
        // lambda not seeded here)
        const bool shape_ok = pl.cnot ? (pp.diag >= 0 && ((pp.rotA >= 0 && pp.rotB < 0) ||
                                                          (pp.gather && pp.rotA < 0 && pp.rotB >= 0)))
                                      : (pp.rotA >= 0 && pp.diag >= 0 && pp.rotB >= 0);
        if (c->half && !pp.init && shape_ok && !(extra_flags & (PF_FUSED | PF_SEED))) {
            a.flags |= PF_HALF;
            a.hview = c->hviews + pp.view;
        }
        // lambda goes back through the chain's index map: other tiles still read the
        // old lambda, so the pass writes the second buffer and the two swap roles
        if (pl.cnot && pp.gather) a.psi_out = c->lam_alt;
    }
    const int rc = run_on(c, st, HQML_K_BWD_PASS, "backward pass launch",
                          [&] { return launch_tile_bwd(a, sp.bc, c->cfg.storage, c->r64, st); });
    if (rc == HQML_OK && (a.flags & PF_GATHER)) std::swap(c->lam, c->lam_alt);
    return rc;
}

int prep(hqml_ctx *c, int B, const void *x, const void *theta, int io64)
{
    return run(c, HQML_K_OTHER, "table preparation", [&] {
        const int ent = c->cfg.entangler != HQML_ENT_CNOT ? 0 : c->plan.small ? 1 : 2;
        return launch_prep(theta, x, io64, c->plan.L, c->plan.n, B, c->zyz, c->frame, c->rot_tf, c->dw, c->H,
                           c->init_u, ent, c->r64, c->stream);
    });
}

// The Pauli string the tile passes measure.  The CNOT-chain plan stops before the last
// chain P, so it measures P^dag O P: X^x -> X^(x ^ (x << 1)) and Z^z -> Z^z' (bit k of z'
// = parity of bits k.. of z), and O = i^|x & z| X^x Z^z becomes s i^|x' & z'| X^x' Z^z'
// with the sign s = i^(|x & z| - |x' & z'|) = +-1.
struct ObsString {
    uint32_t z, x;
    bool neg;
};

ObsString tile_observable(const hqml_config *cfg, const Plan &plan)
{
    ObsString o;
    o.z = (cfg->obs_mask | cfg->obs_x_mask) ? (uint32_t)cfg->obs_mask : 1u;
    o.x = (uint32_t)cfg->obs_x_mask;
    o.neg = false;
    if (!plan.cnot) return o;
    const uint32_t full = (uint32_t)((1ull << plan.n) - 1ull);
    const int d0 = __builtin_popcount(o.z & o.x);
    uint32_t z = o.z;
    for (int sh = 1; sh < 32; sh <<= 1) z ^= z >> sh;
    o.z = z;
    o.x = (o.x ^ (o.x << 1)) & full;
    const int d = d0 - __builtin_popcount(o.z & o.x);
    o.neg = (((d % 4) + 4) % 4) == 2;
    return o;
}

int check_config(const hqml_config *cfg, Plan *plan, std::string *err)
{
    if (!cfg) {
        *err = "cfg is NULL";
        return HQML_ERR_ARG;
    }
    if (cfg->max_batch < 1) {
        *err = "max_batch must be >= 1";
        return HQML_ERR_ARG;
    }
    if (cfg->storage != HQML_STORE_FP32 && cfg->storage != HQML_STORE_BF16 && cfg->storage != HQML_STORE_FP64) {
        *err = "storage must be HQML_STORE_FP32, HQML_STORE_BF16 or HQML_STORE_FP64";
        return HQML_ERR_ARG;
    }
    if (cfg->compute != HQML_COMPUTE_FP32 && cfg->compute != HQML_COMPUTE_FP64) {
        *err = "compute must be HQML_COMPUTE_FP32 or HQML_COMPUTE_FP64";
        return HQML_ERR_ARG;
    }
    if ((cfg->storage == HQML_STORE_FP64 && cfg->compute != HQML_COMPUTE_FP64) ||
        (cfg->storage == HQML_STORE_BF16 && cfg->compute != HQML_COMPUTE_FP32)) {
        *err = "fp64 storage needs fp64 compute; bf16 storage needs fp32 compute";
        return HQML_ERR_UNSUPPORTED;
    }
    if (cfg->compute == HQML_COMPUTE_FP64 && cfg->n_qubits == 13) {
        *err = "fp64 compute supports n_qubits <= 12 (whole circuit per workgroup) or >= 14 (tiles)";
        return HQML_ERR_UNSUPPORTED;
    }
    if (cfg->obs_mask < 0 || cfg->obs_x_mask < 0 ||
        (cfg->n_qubits >= 1 && cfg->n_qubits < 31 && ((cfg->obs_mask | cfg->obs_x_mask) >> cfg->n_qubits) != 0)) {
        *err = "obs_mask and obs_x_mask may only name qubits 0..n_qubits-1";
        return HQML_ERR_ARG;
    }
    if (cfg->fusion != HQML_FUSED && cfg->fusion != HQML_GATE_BY_GATE) {
        *err = "fusion must be HQML_FUSED or HQML_GATE_BY_GATE";
        return HQML_ERR_ARG;
    }
    if (cfg->fusion == HQML_GATE_BY_GATE && cfg->max_batch > 65535) {
        *err = "the gate-by-gate comparator takes at most 65535 samples";
        return HQML_ERR_ARG;
    }
    if (cfg->fusion == HQML_GATE_BY_GATE &&
        (cfg->storage != HQML_STORE_FP32 || cfg->compute != HQML_COMPUTE_FP32 || cfg->ckpt_block != 0)) {
        *err = "the gate-by-gate comparator supports fp32 storage and compute without checkpointing only";
        return HQML_ERR_UNSUPPORTED;
    }
    if (cfg->entangler != HQML_ENT_CZ && cfg->entangler != HQML_ENT_CNOT) {
        *err = "entangler must be HQML_ENT_CZ or HQML_ENT_CNOT";
        return HQML_ERR_ARG;
    }
    const bool cnot_tiles = cfg->entangler == HQML_ENT_CNOT && cfg->fusion == HQML_FUSED;
    if (!make_plan(cfg->n_qubits, cfg->n_layers, cfg->ckpt_block, plan, err, cnot_tiles)) return HQML_ERR_ARG;
    if (cfg->obs_x_mask != 0 && !plan->small && cfg->fusion == HQML_FUSED) {
        const ObsString o = tile_observable(cfg, *plan);
        ViewDev ov;
        if (!make_obs_view(cfg->n_qubits, o.x, &ov, err)) return HQML_ERR_UNSUPPORTED;
    }
    if (!plan->small && (size_t)cfg->max_batch * plan->T > 0x7FFFFFFFull) {
        *err = "max_batch * tiles per sample exceeds the grid limit";
        return HQML_ERR_ARG;
    }
    return HQML_OK;
}

// Forward sweep of the tile path for one chunk.  'fuse_last' leaves the last pass to
// the backward sweep.
int tile_forward_sweep(hqml_ctx *c, hipStream_t st, Span sp, bool fuse_last)
{
    const Plan &pl = c->plan;
    const int P = pl.n_fwd();
    const int last = fuse_last ? P - 1 : P;
    for (int p = 0; p < last; ++p) {
        const int rc = fwd_pass(c, st, sp, p, (!fuse_last && p == P - 1 && !c->obs_x) ? PF_EMIT_E : 0);
        if (rc) return rc;
    }
    return HQML_OK;
}

// Backward sweep of the tile path for one chunk.  The last forward pass is either
// fused here (train_step: forward ops, E, seed, adjoint ops in one kernel) or seeded
// from its saved output.  Ends with the per-sample statistics of the chunk in S.
// How the backward sweep starts.
enum LastPass {
    SEED_FROM_SAVED = 0,   // lambda = O psi formed in the first adjoint pass from the saved final state
    FUSED_LAST = 1,        // last forward pass, E, seed and first adjoint pass in one kernel
    LAMBDA_READY = 2       // lambda already holds O psi (written by the observable pass)
};

// Observable pass of a Pauli string with X/Y factors on the final state of a chunk.
int obs_pass(hqml_ctx *c, hipStream_t st, Span sp, int flags)
{
    const Plan &pl = c->plan;
    TilePassArgs a = base_args(c);
    a.lam = c->lam_buf[0];   // the buffer every backward sweep starts from
    a.view = c->views + pl.V;
    a.psi_in = pass_out(c, pl.n_fwd() - 1);
    a.rotA = a.diag = a.rotB = -1;
    a.flags = flags | (pl.cnot ? PF_CNOT : 0) | (c->obs_neg ? PF_OBS_NEG : 0);
    a.sample0 = sp.b0;
    return run_on(c, st, HQML_K_OTHER, "observable pass launch",
                  [&] { return launch_tile_obs(a, sp.bc, c->cfg.storage, c->r64, st); });
}

int tile_backward_sweep(hqml_ctx *c, hipStream_t st, Span sp, int start)
{
    // A CNOT-plan sweep swaps the lambda buffers once per scattering pass; the next
    // chunk's sweep (its seed written by an observable pass queued before this sweep)
    // must start from lam_buf[0] again.
    c->lam = c->lam_buf[0];
    c->lam_alt = c->lam_buf[1];
    const int last_flags = start == FUSED_LAST ? (PF_FUSED | PF_EMIT_E) : start == SEED_FROM_SAVED ? PF_SEED : 0;
    const Plan &pl = c->plan;
    const int P = pl.n_fwd();
    const int nso = (int)pl.stats_only.size();
    int rc;
    const int2 *map = c->statmap;
    auto reduce = [&](const char *base, int lo, int hi) {
        return run_on(c, st, HQML_K_OTHER, "statistics reduction", [&] {
            return launch_stats_reduce(base, c->r64, map, sp.bs, sp.b0, sp.bc, pl.L, pl.n, pl.T * c->stat_mul, lo,
                                       hi, c->S, c->part2, st);
        });
    };
    if (pl.c == 0) {
        for (int k = P - 1; k >= 0; --k) {
            int fl = 0;
            if (k == P - 1) fl = last_flags;
            if ((rc = bwd_pass(c, st, sp, k, 0, c->part, fl))) return rc;
        }
        for (int i = 0; i < nso; ++i)
            if ((rc = bwd_pass(c, st, sp, P + i, 0, c->part, 0))) return rc;
        return reduce(c->part, 0, P + nso);
    }
    for (int k = pl.nblocks - 1; k >= 0; --k) {
        const int lo = k * pl.c, hi = std::min(P, lo + pl.c);
        if (k < pl.nblocks - 1) {
            for (int p = lo; p < hi - 1; ++p)
                if ((rc = fwd_pass(c, st, sp, p, 0))) return rc;
        }
        for (int p = hi - 1; p >= lo; --p) {
            int fl = 0;
            if (p == P - 1) fl = last_flags;
            if ((rc = bwd_pass(c, st, sp, p, lo, c->part, fl))) return rc;
        }
        if ((rc = reduce(c->part, lo, hi))) return rc;
    }
    char *so_base = c->part + (size_t)pl.c * sp.bs * pl.T * c->stat_mul * kSlots * c->rb;
    for (int i = 0; i < nso; ++i)
        if ((rc = bwd_pass(c, st, sp, P + i, P, so_base, 0))) return rc;
    if (nso > 0) return reduce(so_base, P, P + nso);
    return HQML_OK;
}

// Number of batch chunks for a training step on the tile path.
int chunk_count(const hqml_ctx *c, int B)
{
    if (c->timing || !c->aux) return 1;
    // Default: two chunks when the backward sweep recomputes checkpoint blocks (the next
    // chunk's forward passes fill the gaps; 1000 layers, checkpoint every 20: +5 %),
    // one otherwise (20 qubits, 100 layers, every pass output kept: one chunk is 1 %
    // faster, the pipeline's smaller grids costing more than the overlap gains).
    int C = c->chunks > 0 ? c->chunks : (c->plan.c > 0 ? 2 : 1);
    C = std::min(C, std::min(B, 8));
    while (C > 1 && (long long)(B / C) * c->plan.T < 256) --C;   // keep >= 256 workgroups a chunk
    return std::max(C, 1);
}

SmallArgs small_args(hqml_ctx *c, int mode)
{
    SmallArgs a;
    std::memset(&a, 0, sizeof a);
    a.init_u = c->init_u;
    a.rot_tf = c->rot_tf;
    a.dw = c->dw;
    a.psi_save = reinterpret_cast<float *>(c->saved);
    a.e_out = c->e_part;
    a.stats = c->S;
    a.n = c->plan.n;
    a.L = c->plan.L;
    a.mode = mode;
    a.ent = c->cfg.entangler;
    a.obs = c->obs;
    a.obs_x = c->obs_x;
    return a;
}

// ---- gate-by-gate comparator ----

Workspace workspace_for(const hqml_config *cfg, const Plan &plan)
{
    if (cfg->fusion == HQML_GATE_BY_GATE) return size_workspace_gbg(plan.n, plan.L, cfg->max_batch);
    return size_workspace(plan, cfg->max_batch, cfg->storage, cfg->compute == HQML_COMPUTE_FP64);
}

int gbg_forward_sweep(hqml_ctx *c, int B, const float *x, const float *theta)
{
    const int n = c->plan.n, L = c->plan.L;
    const bool cnot = c->cfg.entangler == HQML_ENT_CNOT;
    float2 *psi = reinterpret_cast<float2 *>(c->gbg_psi);
    int rc = run(c, HQML_K_OTHER, "theta copy",
                 [&] { return launch_gbg_copy(theta, L * n * 3, c->gbg_theta, c->stream); });
    if (rc) return rc;
    if ((rc = run(c, HQML_K_GATE, "state initialisation", [&] { return launch_gbg_zero(psi, n, B, c->stream); })))
        return rc;
    for (int q = 0; q < n; ++q)   // encoding Ry(x[b][q])
        if ((rc = run(c, HQML_K_GATE, "encoding gate",
                      [&] { return launch_gbg_rot(1, psi, n, B, q, x + q, n, c->stream); })))
            return rc;
    for (int l = 0; l < L; ++l) {
        for (int q = 0; q < n; ++q)
            for (int g = 0; g < 3; ++g)
                if ((rc = run(c, HQML_K_GATE, "rotation gate", [&] {
                         return launch_gbg_rot(g, psi, n, B, q, c->gbg_theta + ((size_t)l * n + q) * 3 + g, 0,
                                               c->stream);
                     })))
                    return rc;
        for (int q = 0; q + 1 < n; ++q)
            if ((rc = run(c, HQML_K_GATE, "entangling gate", [&] {
                     return cnot ? launch_gbg_cnot(psi, nullptr, n, B, q, c->stream)
                                 : launch_gbg_cz(psi, nullptr, n, B, q, c->stream);
                 })))
                return rc;
    }
    return run(c, HQML_K_GATE, "<O> partials",
               [&] { return launch_gbg_expz(psi, n, B, c->obs, c->obs_x, static_cast<float *>(c->e_part), c->stream); });
}

// Adjoint sweep from the final state left in gbg_psi; leaves the gradient block sums
// in gbg_part and psi un-computed back to the encoded state.
int gbg_backward_sweep(hqml_ctx *c, int B)
{
    const int n = c->plan.n, L = c->plan.L;
    const bool cnot = c->cfg.entangler == HQML_ENT_CNOT;
    float2 *psi = reinterpret_cast<float2 *>(c->gbg_psi);
    float2 *lam = reinterpret_cast<float2 *>(c->gbg_lam);
    const size_t per_gate = (size_t)B * c->gbg_blocks;
    int rc = run(c, HQML_K_GATE, "adjoint seed",
                 [&] { return launch_gbg_seed(psi, lam, n, B, c->obs, c->obs_x, c->stream); });
    if (rc) return rc;
    for (int l = L - 1; l >= 0; --l) {
        for (int q = n - 2; q >= 0; --q)   // self-inverse gates, undone in reverse order
            if ((rc = run(c, HQML_K_GATE, "entangling gate adjoint", [&] {
                     return cnot ? launch_gbg_cnot(psi, lam, n, B, q, c->stream) : launch_gbg_cz(psi, lam, n, B, q, c->stream);
                 })))
                return rc;
        for (int q = n - 1; q >= 0; --q)
            for (int g = 2; g >= 0; --g) {
                const size_t p = ((size_t)l * n + q) * 3 + g;
                if ((rc = run(c, HQML_K_GATE, "rotation adjoint", [&] {
                         return launch_gbg_rot_adj(g, psi, lam, n, B, q, c->gbg_theta + p, c->gbg_part + p * per_gate,
                                                   c->stream);
                     })))
                    return rc;
            }
    }
    return HQML_OK;
}

int gbg_grad(hqml_ctx *c, int B, float *grad)
{
    const Plan &pl = c->plan;
    return run(c, HQML_K_OTHER, "gradient reduction", [&] {
        return launch_gbg_grad(c->gbg_part, c->dlde, B, pl.n, pl.L * pl.n * 3, grad, c->stream);
    });
}

}  // namespace

namespace hqml {

int validate_config(const hqml_config *cfg, Plan *plan, std::string *err)
{
    return check_config(cfg, plan, err);
}

// Memory this library's kernels can read or write: device memory of `device`, managed
// memory, or pinned host memory mapped into the device; pageable host memory is
// refused, as is an array that runs past the end of the allocation that holds it (for a
// sub-allocator such as PyTorch's caching allocator, the runtime's allocation is the
// whole segment).
int check_device_array(int device, const void *p, size_t bytes, const char *name, std::string *err,
                       const void **base_out, size_t *size_out)
{
    if (!p) {
        *err = std::string(name) + " is NULL";
        return HQML_ERR_ARG;
    }
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();   // the failed query leaves its error behind
        *err = std::string(name) + " is not memory known to HIP";
        return HQML_ERR_ARG;
    }
    const bool on_device = at.type == hipMemoryTypeDevice && at.device == device;
    const bool mapped = (at.type == hipMemoryTypeHost || at.type == hipMemoryTypeManaged) && at.devicePointer == p;
    if (!on_device && !mapped) {
        *err = std::string(name) + " must be device memory of the context's device "
                                   "(or pinned host memory), not pageable host memory";
        return HQML_ERR_ARG;
    }
    void *base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) != hipSuccess) {
        (void)hipGetLastError();
        *err = std::string(name) + ": allocation range unknown";
        return HQML_ERR_ARG;
    }
    const size_t room = static_cast<size_t>(static_cast<const char *>(base) + size - static_cast<const char *>(p));
    if (bytes > room) {
        *err = std::string(name) + " needs " + std::to_string(bytes) + " bytes, its allocation has " +
               std::to_string(room) + " from that address";
        return HQML_ERR_ARG;
    }
    if (base_out) *base_out = base;
    if (size_out) *size_out = size;
    return HQML_OK;
}

void set_thread_error(const std::string &msg)
{
    g_create_err = msg;
}

void config_observable(const hqml_config *cfg, const Plan &plan, uint32_t *z, uint32_t *x, bool *neg)
{
    const ObsString o = tile_observable(cfg, plan);
    *z = o.z;
    *x = o.x;
    *neg = o.neg;
}

}  // namespace hqml

extern "C" {

size_t hqml_workspace_bytes(const hqml_config *cfg)
{
    Plan plan;
    std::string err;
    if (check_config(cfg, &plan, &err) != HQML_OK) return 0;
    return workspace_for(cfg, plan).total;
}

long long hqml_describe_plan(const hqml_config *cfg, char *buf, size_t len)
{
    Plan plan;
    std::string err;
    const int rc = check_config(cfg, &plan, &err);
    if (rc != HQML_OK) return rc;
    std::string s;
    if (cfg->fusion == HQML_GATE_BY_GATE) {
        char tmp[128];
        std::snprintf(tmp, sizeof tmp, "{\"n\": %d, \"L\": %d, \"gate_by_gate\": true, \"blocks\": %d}", plan.n,
                      plan.L, gbg_blocks_per_sample(plan.n));
        s = tmp;
    } else {
        s = describe_plan(plan);
    }
    if (buf && len > 0) {
        const size_t k = std::min(len - 1, s.size());
        std::memcpy(buf, s.data(), k);
        buf[k] = '\0';
    }
    return (long long)s.size();
}

int hqml_create(const hqml_config *cfg, hqml_ctx **out)
{
    if (!out) return fail(nullptr, HQML_ERR_ARG, "out is NULL");
    *out = nullptr;
    Plan plan;
    std::string err;
    int rc = check_config(cfg, &plan, &err);
    if (rc != HQML_OK) return fail(nullptr, rc, err);
    hqml_ctx *c = new (std::nothrow) hqml_ctx;
    if (!c) return fail(nullptr, HQML_ERR_OOM, "host allocation failed");
    c->cfg = *cfg;
    c->plan = plan;
    c->gbg = cfg->fusion == HQML_GATE_BY_GATE;
    c->r64 = cfg->compute == HQML_COMPUTE_FP64 ? 1 : 0;
    c->rb = c->r64 ? 8 : 4;
    {
        const ObsString o = tile_observable(cfg, plan);
        c->obs = o.z;
        c->obs_x = o.x;
        c->obs_neg = o.neg;
    }
    c->ws = workspace_for(cfg, plan);
    c->stream = reinterpret_cast<hipStream_t>(cfg->stream);
    hipError_t e = hipSetDevice(cfg->device);
    if (e != hipSuccess) {
        delete c;
        return fail(nullptr, HQML_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
    }
    size_t free_b = 0, total_b = 0;
    e = hipMemGetInfo(&free_b, &total_b);
    if (e != hipSuccess) {
        delete c;
        return fail(nullptr, HQML_ERR_HIP, std::string("hipMemGetInfo: ") + hipGetErrorString(e));
    }
    if (c->ws.total > free_b) {
        char msg[160];
        std::snprintf(msg, sizeof msg, "workspace needs %zu bytes, device has %zu free", c->ws.total, free_b);
        delete c;
        return fail(nullptr, HQML_ERR_OOM, msg);
    }
    const int B = cfg->max_batch;
    const size_t Ln = (size_t)plan.L * plan.n;
    bool ok = true;
    auto grab = [&](size_t bytes) -> void * {
        if (!ok || bytes == 0) return nullptr;
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) {
            ok = false;
            return nullptr;
        }
        c->allocs.push_back(p);
        return p;
    };
    if (c->gbg) {
        const int nblk = gbg_blocks_per_sample(plan.n);
        c->gbg_blocks = nblk;
        c->gbg_psi = static_cast<float *>(grab(c->ws.state_bytes));
        c->gbg_lam = static_cast<float *>(grab(c->ws.lam_bytes));
        c->gbg_part = static_cast<double *>(grab(c->ws.part_bytes));
        c->gbg_theta = static_cast<float *>(grab(Ln * 3 * 4));
        c->e_part = grab((size_t)B * nblk * 4);
        c->dlde = static_cast<double *>(grab((size_t)B * 8));
        c->e_work = static_cast<double *>(grab((size_t)B * 8));
        c->epart2 = static_cast<double *>(grab(c->ws.epart2_bytes));
        c->loss_tmp = static_cast<float *>(grab(64));
        if (!ok) {
            hqml_destroy(c);
            return fail(nullptr, HQML_ERR_OOM, "hipMalloc failed while reserving the workspace");
        }
        *out = c;
        return HQML_OK;
    }
    c->saved = static_cast<char *>(grab((size_t)c->ws.n_saved * c->ws.state_bytes));
    c->lam = grab(c->ws.lam_bytes);
    if (plan.cnot) c->lam_alt = grab(c->ws.lam_bytes);
    c->lam_buf[0] = c->lam;
    c->lam_buf[1] = c->lam_alt;
    c->part = static_cast<char *>(grab(c->ws.part_bytes));
    c->e_part = grab((size_t)B * plan.T * c->rb);
    c->S = static_cast<double *>(grab((size_t)B * Ln * 3 * 8));
    c->zyz = static_cast<double *>(grab(Ln * 6 * 8));
    c->frame = static_cast<unsigned char *>(grab(Ln));
    c->rot_tf = grab(Ln * 2 * c->rb);
    c->dw = grab(Ln * 4 * c->rb * (plan.cnot ? 2 : 1));   // CNOT tiles: diag(p_l) and diag(r_l) rows
    c->H = static_cast<double *>(grab(Ln * 9 * 8));
    c->init_u = grab((size_t)B * plan.n * 4 * c->rb);
    if (!plan.small) c->views = static_cast<ViewDev *>(grab((plan.views.size() + 1) * sizeof(ViewDev)));
    c->half = !plan.small && plan.half;
    c->stat_mul = plan.small ? 1 : stat_tiles(plan, c->r64) / plan.T;
    if (c->half) c->hviews = static_cast<ViewDevH *>(grab(plan.hviews.size() * sizeof(ViewDevH)));
    c->statmap = static_cast<int2 *>(grab(Ln * sizeof(int2)));
    c->dlde = static_cast<double *>(grab((size_t)B * 8));
    c->e_work = static_cast<double *>(grab((size_t)B * 8));
    c->part2 = static_cast<double *>(grab(c->ws.part2_bytes));
    c->epart2 = static_cast<double *>(grab(c->ws.epart2_bytes));
    c->loss_tmp = static_cast<float *>(grab(64));
    if (!ok) {
        hqml_destroy(c);
        return fail(nullptr, HQML_ERR_OOM, "hipMalloc failed while reserving the workspace");
    }
    std::vector<int2> sm(Ln);
    for (size_t i = 0; i < Ln; ++i) sm[i] = make_int2(plan.statmap[i].pass, plan.statmap[i].slot);
    e = hipMemcpy(c->statmap, sm.data(), Ln * sizeof(int2), hipMemcpyHostToDevice);
    if (e == hipSuccess && !plan.small) {
        std::vector<ViewDev> vs(plan.views);
        ViewDev ov;
        std::memset(&ov, 0, sizeof(ov));
        std::string verr;
        if (c->obs_x && !make_obs_view(plan.n, c->obs_x, &ov, &verr)) {
            hqml_destroy(c);
            return fail(nullptr, HQML_ERR_UNSUPPORTED, verr);
        }
        vs.push_back(ov);   // views[V]: the observable pass (unused without X/Y factors)
        e = hipMemcpy(c->views, vs.data(), vs.size() * sizeof(ViewDev), hipMemcpyHostToDevice);
        if (e == hipSuccess && c->half)
            e = hipMemcpy(c->hviews, plan.hviews.data(), plan.hviews.size() * sizeof(ViewDevH), hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && plan.small) e = configure_small();
    if (e != hipSuccess) {
        const std::string m = std::string("workspace set-up: ") + hipGetErrorString(e);
        hqml_destroy(c);
        return fail(nullptr, HQML_ERR_HIP, m);
    }
    if (!plan.small) {
        e = hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_start, hipEventDisableTiming);
        for (int k = 0; k < 8 && e == hipSuccess; ++k) e = hipEventCreateWithFlags(&c->ev_fwd[k], hipEventDisableTiming);
        if (e != hipSuccess) {
            const std::string m = std::string("stream set-up: ") + hipGetErrorString(e);
            hqml_destroy(c);
            return fail(nullptr, HQML_ERR_HIP, m);
        }
    }
    *out = c;
    return HQML_OK;
}

int hqml_destroy(hqml_ctx *c)
{
    if (!c) return HQML_OK;
    (void)hipSetDevice(c->cfg.device);
    (void)hipStreamSynchronize(c->stream);
    if (c->aux) {
        (void)hipStreamSynchronize(c->aux);
        (void)hipStreamDestroy(c->aux);
    }
    if (c->ev_start) (void)hipEventDestroy(c->ev_start);
    for (hipEvent_t e : c->ev_fwd)
        if (e) (void)hipEventDestroy(e);
    for (void *p : c->allocs) (void)hipFree(p);
    for (hipEvent_t e : c->pool) (void)hipEventDestroy(e);
    delete c;
    return HQML_OK;
}

}  // extern "C"

namespace {

int forward_impl(hqml_ctx *c, int B, const void *x, const void *theta, void *expz, int save_for_backward, int io64)
{
    if (!c) return HQML_ERR_ARG;
    c->err.clear();
    if (B < 0 || B > c->cfg.max_batch) return fail(c, HQML_ERR_ARG, "B must be in 0..max_batch");
    c->saved_B = -1;
    if (B == 0) {
        if (save_for_backward) c->saved_B = 0;
        return HQML_OK;
    }
    hipError_t e = hipSetDevice(c->cfg.device);
    if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
    const size_t io = io64 ? sizeof(double) : sizeof(float), nq = (size_t)c->cfg.n_qubits;
    int rc;
    if ((rc = check_array(c, 0, x, (size_t)B * nq * io, "x")) ||
        (rc = check_array(c, 1, theta, (size_t)c->cfg.n_layers * nq * 3 * io, "theta")) ||
        (rc = check_array(c, 3, expz, (size_t)B * io, "expz")))
        return rc;
    if (c->gbg) {
        if ((rc = gbg_forward_sweep(c, B, static_cast<const float *>(x), static_cast<const float *>(theta)))) return rc;
        rc = run(c, HQML_K_OTHER, "E reduction", [&] {
            return launch_ez_reduce(c->e_part, 0, B, c->gbg_blocks, nullptr, expz, nullptr, io64, nullptr,
                                    c->e_work, c->epart2, c->stream);
        });
        if (rc) return rc;
        if (save_for_backward) c->saved_B = B;
        return HQML_OK;
    }
    rc = prep(c, B, x, theta, io64);
    if (rc) return rc;
    const Plan &pl = c->plan;
    if (pl.small) {
        const SmallArgs a = small_args(c, 0);
        if ((rc = run(c, HQML_K_SMALL, "small-circuit kernel", [&] { return launch_small(a, B, c->r64, c->stream); })))
            return rc;
        rc = run(c, HQML_K_OTHER, "E reduction", [&] {
            return launch_ez_reduce(c->e_part, c->r64, B, 1, nullptr, expz, nullptr, io64, nullptr, c->e_work,
                                    c->epart2, c->stream);
        });
    } else {
        if ((rc = tile_forward_sweep(c, c->stream, Span{0, B, B}, false))) return rc;
        c->tail_valid = true;
        if (c->obs_x && (rc = obs_pass(c, c->stream, Span{0, B, B}, PF_EMIT_E))) return rc;
        rc = run(c, HQML_K_OTHER, "E reduction", [&] {
            return launch_ez_reduce(c->e_part, c->r64, B, pl.T, nullptr, expz, nullptr, io64, nullptr, c->e_work,
                                    c->epart2, c->stream);
        });
    }
    if (rc) return rc;
    if (save_for_backward) c->saved_B = B;
    return HQML_OK;
}

// The last checkpoint block's forward passes again, from the checkpoint before it, when
// an earlier backward sweep has overwritten their saved outputs.
int restore_tail_block(hqml_ctx *c, Span sp)
{
    const Plan &pl = c->plan;
    if (pl.c == 0 || pl.nblocks < 2 || c->tail_valid) return HQML_OK;
    const int P = pl.n_fwd();
    for (int p = (pl.nblocks - 1) * pl.c; p < P; ++p) {
        const int rc = fwd_pass(c, c->stream, sp, p, 0);
        if (rc) return rc;
    }
    c->tail_valid = true;
    return HQML_OK;
}

int backward_impl(hqml_ctx *c, const void *dL_dE, void *grad, int io64)
{
    if (!c) return HQML_ERR_ARG;
    c->err.clear();
    hipError_t e = hipSetDevice(c->cfg.device);
    if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
    const size_t io = io64 ? sizeof(double) : sizeof(float);
    int rc = check_array(c, 5, grad, (size_t)c->cfg.n_layers * c->cfg.n_qubits * 3 * io, "grad");
    if (rc) return rc;
    if (c->saved_B < 0) return fail(c, HQML_ERR_STATE, "no saved forward pass on this context");
    const int B = c->saved_B;
    const Plan &pl = c->plan;
    if (B == 0) {  // empty batch: the gradient is zero (the reduction over no samples)
        if (c->gbg) return gbg_grad(c, 0, static_cast<float *>(grad));
        return run(c, HQML_K_OTHER, "gradient reduction", [&] {
            return launch_grad_reduce(c->S, c->H, c->dlde, 0, pl.L, pl.n, grad, io64, c->stream);
        });
    }
    if ((rc = check_array(c, 6, dL_dE, (size_t)B * io, "dL_dE"))) return rc;
    rc = run(c, HQML_K_OTHER, "dL/dE copy", [&] { return launch_copy_dlde(dL_dE, io64, B, c->dlde, c->stream); });
    if (rc) return rc;
    if (c->gbg) {
        c->saved_B = -1;   // the adjoint sweep un-computes the saved state in place
        if ((rc = gbg_backward_sweep(c, B))) return rc;
        return gbg_grad(c, B, static_cast<float *>(grad));
    }
    if (pl.small) {
        const SmallArgs a = small_args(c, 1);
        rc = run(c, HQML_K_SMALL, "small-circuit kernel", [&] { return launch_small(a, B, c->r64, c->stream); });
    } else {
        if ((rc = restore_tail_block(c, Span{0, B, B}))) return rc;
        if (c->obs_x && (rc = obs_pass(c, c->stream, Span{0, B, B}, PF_SEED))) return rc;
        rc = tile_backward_sweep(c, c->stream, Span{0, B, B}, c->obs_x ? LAMBDA_READY : SEED_FROM_SAVED);
        if (pl.c > 0 && pl.nblocks > 1) c->tail_valid = false;   // the sweep recomputed other blocks
    }
    if (rc) return rc;
    return run(c, HQML_K_OTHER, "gradient reduction", [&] {
        return launch_grad_reduce(c->S, c->H, c->dlde, B, pl.L, pl.n, grad, io64, c->stream);
    });
}

int train_impl(hqml_ctx *c, int B, const void *x, const void *theta, const void *y, void *expz, void *loss,
               void *grad, int io64)
{
    if (!c) return HQML_ERR_ARG;
    c->err.clear();
    if (B < 1 || B > c->cfg.max_batch) return fail(c, HQML_ERR_ARG, "B must be in 1..max_batch");
    hipError_t e = hipSetDevice(c->cfg.device);
    if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
    const size_t io = io64 ? sizeof(double) : sizeof(float), nq = (size_t)c->cfg.n_qubits;
    const size_t np = (size_t)c->cfg.n_layers * nq * 3 * io;
    int rc;
    if ((rc = check_array(c, 0, x, (size_t)B * nq * io, "x")) || (rc = check_array(c, 1, theta, np, "theta")) ||
        (rc = check_array(c, 2, y, (size_t)B * io, "y")) || (rc = check_array(c, 3, expz, (size_t)B * io, "expz")) ||
        (rc = check_array(c, 4, loss, io, "loss")) || (rc = check_array(c, 5, grad, np, "grad")))
        return rc;
    c->saved_B = -1;
    if (c->gbg) {
        if ((rc = gbg_forward_sweep(c, B, static_cast<const float *>(x), static_cast<const float *>(theta)))) return rc;
        rc = run(c, HQML_K_OTHER, "E reduction", [&] {
            return launch_ez_reduce(c->e_part, 0, B, c->gbg_blocks, y, expz, loss, io64, c->dlde, c->e_work,
                                    c->epart2, c->stream);
        });
        if (rc) return rc;
        if ((rc = gbg_backward_sweep(c, B))) return rc;
        return gbg_grad(c, B, static_cast<float *>(grad));
    }
    rc = prep(c, B, x, theta, io64);
    if (rc) return rc;
    const Plan &pl = c->plan;
    if (pl.small) {
        const SmallArgs a = small_args(c, 2);
        if ((rc = run(c, HQML_K_SMALL, "small-circuit kernel", [&] { return launch_small(a, B, c->r64, c->stream); })))
            return rc;
        return run(c, HQML_K_OTHER, "E and gradient reduction", [&] {
            return launch_small_reduce(c->e_part, c->r64, B, y, expz, loss, io64, c->dlde, c->S, c->H, pl.L, pl.n, grad,
                                       c->stream);
        });
    } else {
        // The fused last pass emits E; the loss and dL/dE are needed only by the final
        // gradient reduction, so the E reduction runs after the backward sweeps.
        const int C = chunk_count(c, B);
        // the last forward pass is fused with the first backward pass unless lambda comes
        // from the observable pass or the plan has no fused-last shape (CNOT chain)
        const bool fuse = !c->obs_x && !pl.cnot;
        const int start = c->obs_x ? LAMBDA_READY : fuse ? FUSED_LAST : SEED_FROM_SAVED;
        if (C == 1) {
            if ((rc = tile_forward_sweep(c, c->stream, Span{0, B, B}, fuse))) return rc;
            if (c->obs_x && (rc = obs_pass(c, c->stream, Span{0, B, B}, PF_EMIT_E | PF_SEED))) return rc;
            if ((rc = tile_backward_sweep(c, c->stream, Span{0, B, B}, start))) return rc;
        } else {
            hipError_t he = hipEventRecord(c->ev_start, c->stream);
            if (he == hipSuccess) he = hipStreamWaitEvent(c->aux, c->ev_start, 0);
            if (he != hipSuccess) return hip_fail(c, he, "stream ordering");
            std::vector<Span> spans;
            for (int k = 0; k < C; ++k) {
                const int b0 = (int)((long long)B * k / C), b1 = (int)((long long)B * (k + 1) / C);
                spans.push_back(Span{b0, b1 - b0, B});
            }
            for (int k = 0; k < C; ++k) {
                if ((rc = tile_forward_sweep(c, c->aux, spans[k], fuse))) return rc;
                if (c->obs_x && (rc = obs_pass(c, c->aux, spans[k], PF_EMIT_E | PF_SEED))) return rc;
                he = hipEventRecord(c->ev_fwd[k], c->aux);
                if (he != hipSuccess) return hip_fail(c, he, "stream ordering");
            }
            for (int k = 0; k < C; ++k) {
                he = hipStreamWaitEvent(c->stream, c->ev_fwd[k], 0);
                if (he != hipSuccess) return hip_fail(c, he, "stream ordering");
                if ((rc = tile_backward_sweep(c, c->stream, spans[k], start))) return rc;
            }
        }
        rc = run(c, HQML_K_OTHER, "E reduction", [&] {
            return launch_ez_reduce(c->e_part, c->r64, B, pl.T, y, expz, loss, io64, c->dlde, c->e_work,
                                    c->epart2, c->stream);
        });
        if (rc) return rc;
    }
    return run(c, HQML_K_OTHER, "gradient reduction", [&] {
        return launch_grad_reduce(c->S, c->H, c->dlde, B, pl.L, pl.n, grad, io64, c->stream);
    });
}

}  // namespace

extern "C" {

int hqml_forward(hqml_ctx *c, int B, const float *x, const float *theta, float *expz, int save_for_backward)
{
    return forward_impl(c, B, x, theta, expz, save_for_backward, 0);
}

int hqml_backward(hqml_ctx *c, const float *dL_dE, float *grad)
{
    return backward_impl(c, dL_dE, grad, 0);
}

int hqml_train_step(hqml_ctx *c, int B, const float *x, const float *theta, const float *y, float *expz,
                    float *loss, float *grad)
{
    return train_impl(c, B, x, theta, y, expz, loss, grad, 0);
}

int hqml_forward_f64(hqml_ctx *c, int B, const double *x, const double *theta, double *expz, int save_for_backward)
{
    if (c && c->gbg) return fail(c, HQML_ERR_UNSUPPORTED, "the gate-by-gate comparator takes fp32 arrays");
    return forward_impl(c, B, x, theta, expz, save_for_backward, 1);
}

int hqml_backward_f64(hqml_ctx *c, const double *dL_dE, double *grad)
{
    if (c && c->gbg) return fail(c, HQML_ERR_UNSUPPORTED, "the gate-by-gate comparator takes fp32 arrays");
    return backward_impl(c, dL_dE, grad, 1);
}

int hqml_train_step_f64(hqml_ctx *c, int B, const double *x, const double *theta, const double *y, double *expz,
                        double *loss, double *grad)
{
    if (c && c->gbg) return fail(c, HQML_ERR_UNSUPPORTED, "the gate-by-gate comparator takes fp32 arrays");
    return train_impl(c, B, x, theta, y, expz, loss, grad, 1);
}

const char *hqml_status_str(int s)
{
    switch (s) {
    case HQML_OK: return "ok";
    case HQML_ERR_ARG: return "invalid argument";
    case HQML_ERR_OOM: return "out of device memory";
    case HQML_ERR_HIP: return "HIP runtime error";
    case HQML_ERR_STATE: return "call out of order";
    case HQML_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
    }
}

const char *hqml_last_error(const hqml_ctx *c)
{
    return c ? c->err.c_str() : g_create_err.c_str();
}

int hqml_set_timing(hqml_ctx *c, int enable)
{
    if (!c) return HQML_ERR_ARG;
    c->timing = enable != 0;
    return HQML_OK;
}

int hqml_set_overlap(hqml_ctx *c, int chunks)
{
    if (!c) return HQML_ERR_ARG;
    if (chunks < 0 || chunks > 8) return fail(c, HQML_ERR_ARG, "chunks must be in 0..8");
    c->chunks = chunks;
    return HQML_OK;
}

int hqml_kernel_times(hqml_ctx *c, double *ms, long long *count, int reset)
{
    if (!c || !ms || !count) return HQML_ERR_ARG;
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
    for (int k = 0; k < HQML_K_COUNT; ++k) {
        ms[k] = 0.0;
        count[k] = 0;
    }
    for (const auto &r : c->recs) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
            ms[r.kind] += t;
            count[r.kind] += 1;
        }
    }
    if (reset) {
        c->recs.clear();
        c->pool_used = 0;
    }
    return HQML_OK;
}

int hqml_plan_info(const hqml_ctx *c, int *fwd_passes, int *bwd_passes, int *tiles_per_sample,
                   size_t *state_bytes)
{
    if (!c) return HQML_ERR_ARG;
    const Plan &pl = c->plan;
    if (c->gbg) {
        const int gates = pl.L * (4 * pl.n - 1);   // 3n rotations and n-1 entangling gates per layer
        if (fwd_passes) *fwd_passes = gates + pl.n;
        if (bwd_passes) *bwd_passes = gates;
        if (tiles_per_sample) *tiles_per_sample = c->gbg_blocks;
        if (state_bytes) *state_bytes = ((size_t)1 << pl.n) * 8;
        return HQML_OK;
    }
    if (fwd_passes) *fwd_passes = pl.small ? 1 : pl.n_fwd();
    if (bwd_passes) *bwd_passes = pl.small ? 1 : pl.n_bwd();
    if (tiles_per_sample) *tiles_per_sample = pl.T;
    if (state_bytes) *state_bytes = ((size_t)1 << pl.n) * elem_bytes(c);
    return HQML_OK;
}

}  // extern "C"
