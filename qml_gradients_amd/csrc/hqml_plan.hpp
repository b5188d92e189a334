// Host scheduler: views, fused-pass schedule, checkpoint plan and workspace sizes.
// Pure C++ (no HIP calls), so it can size a workspace on a machine without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "hqml_internal.hpp"

namespace hqml {

struct PassPlan {
    int view;
    bool init;    // generates the layer-0 product state (all of Ry-layer 0)
    int rotA;     // Ry-layer applied to the view's group first (-1: none)
    int diag;     // row of the diagonal table applied next (-1: none)
    int rotB;     // Ry-layer applied to the view's group last (-1: none)
    bool gather = false;   // CNOT chain: the input is read through the chain's index map
                           // (and the backward pass writes lambda back through it)
};

struct StatLoc {
    int pass;     // backward pass index (forward passes, then layer-0 stats-only passes)
    int slot;     // (sel*13 + pos)*3
};

struct Plan {
    int n = 0, L = 0;
    bool small = false;                  // n <= 13: whole circuit in one workgroup per sample
    bool cnot = false;                   // tile path with the CNOT-chain entangler
    int V = 0;                           // views (tile path)
    int T = 1;                           // tiles per sample
    std::vector<ViewDev> views;
    std::vector<ViewDevH> hviews;        // half-tile views of the same groups
    bool half = false;                   // every view has a half-tile view: the adjoint passes of
                                         // the general shape (and the CNOT chain's two shapes with a
                                         // diagonal) run on half tiles
    std::vector<PassPlan> fwd;           // forward passes in order
    std::vector<int> stats_only;         // views needing a layer-0 stats-only backward pass
    std::vector<StatLoc> statmap;        // [L*n]
    // checkpointing (tile path): block of c passes; ckpt_block = 0 keeps every output
    int c = 0;                           // passes per block (0: store every pass output)
    int nblocks = 1;

    int n_fwd() const { return (int)fwd.size(); }
    int n_bwd() const { return (int)fwd.size() + (int)stats_only.size(); }
};

// Build the plan for an n-qubit, L-layer circuit; ckpt_block = layers per
// checkpoint block (0 = keep every fused-pass output).  cnot: layers end with the
// CNOT chain instead of the CZ chain (tile path: one pass per view and layer).
// Returns false with a message in *err for unsupported sizes.
bool make_plan(int n, int L, int ckpt_block, Plan *plan, std::string *err, bool cnot = false);

// View for the observable pass of a Pauli string whose X part is xmask: qubits 0..3
// and every higher qubit of xmask on chip (at most 9), the rest as tile bits.
// Returns false with a message for n <= 13 or too many X/Y qubits.
bool make_obs_view(int n, uint32_t xmask, ViewDev *out, std::string *err);

// Device memory layout of a context.
struct Workspace {
    size_t state_elems = 0;     // amplitudes per sample
    size_t state_bytes = 0;     // bytes of one saved state for the whole batch
    size_t lam_bytes = 0;       // adjoint state, fp32
    int n_saved = 0;            // saved-state buffers (pass outputs, or block buffers + checkpoints)
    int n_ckpt = 0;             // of which checkpoints
    int part_passes = 0;        // passes whose statistics partials are held at once
    size_t part_bytes = 0;
    int tile_chunks = 0;        // first-stage reduction blocks per sample (0: tiles summed directly)
    size_t part2_bytes = 0;     // first-stage sums of the statistics partials, fp64
    size_t epart2_bytes = 0;    // first-stage sums of the <O> partials, fp64
    size_t tables_bytes = 0;
    size_t total = 0;
};

// Statistics partials per sample of a backward pass: 2T when the adjoint runs passes on half
// tiles (p.half), else T.
int stat_tiles(const Plan &p, int compute64);

// storage: 0 fp32, 1 bf16, 2 fp64 saved states; compute64: arithmetic (and lambda,
// tables, partial sums) in fp64.
Workspace size_workspace(const Plan &p, int max_batch, int storage, int compute64);

// Gate-by-gate comparator: workgroups per sample of one gate kernel, and its
// workspace (psi and lambda as fp32 states, per-gate fp64 block sums of the
// gradient terms in part_bytes, per-block <O> partials, a copy of theta).
int gbg_blocks_per_sample(int n);
Workspace size_workspace_gbg(int n, int L, int max_batch);

// Human-readable JSON description of a plan (for tests and reports).
std::string describe_plan(const Plan &p);

}  // namespace hqml
