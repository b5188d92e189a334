// Host-side declarations shared by the library's host code (hqml_abi.cpp,
// hqml_noalloc.hip): the kernel launch wrappers of the .hip units and the argument
// checks of the C ABI.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <string>

#include "../../include/hqml.h"
#include "hqml_internal.hpp"
#include "hqml_plan.hpp"

namespace hqml {
// Type codes: io64 = caller arrays are double; r64 = compute in double; storage 0/1/2 =
// fp32 / bf16 / fp64 saved states.
// ent: 0 CZ chain; 1 CNOT chain, whole-circuit tables; 2 CNOT chain, tile tables
hipError_t launch_prep(const void *theta, const void *x, int io64, int L, int n, int B, double *zyz,
                       unsigned char *G, void *rot_tf, void *dw, double *H, void *init_u, int ent, int r64,
                       hipStream_t s);
hipError_t launch_tile_fwd(const TilePassArgs &a, int B, int storage, int r64, hipStream_t s);
hipError_t launch_tile_obs(const TilePassArgs &a, int B, int storage, int r64, hipStream_t s);
hipError_t launch_tile_bwd(const TilePassArgs &a, int B, int storage, int r64, hipStream_t s);
hipError_t launch_small(const SmallArgs &a, int B, int r64, hipStream_t s);
// Allow the whole-circuit kernel (fp32 and fp64 instances, either entangler) the most
// dynamic LDS any supported size needs (two states of 2^13 fp32 or 2^12 fp64
// amplitudes, 128 KiB) on the current device.  Never lowered, so contexts and calls of
// different sizes can interleave.
hipError_t configure_small();
// 12 qubits, CZ chain, fp32 compute: the register-resident whole-circuit kernel
// (hqml_small12.hip), reached through launch_small / configure_small.
hipError_t launch_small12(const SmallArgs &a, int B, hipStream_t s);
hipError_t configure_small12();
hipError_t launch_ez_reduce(const void *e_part, int r64, int B, int T, const void *y, void *e_out, void *loss,
                            int io64, double *dlde, double *e_work, double *chunks, hipStream_t s);
hipError_t launch_copy_dlde(const void *src, int io64, int B, double *dlde, hipStream_t s);
hipError_t launch_stats_reduce(const void *part, int r64, const int2 *map, int Bs, int b0, int Bc, int L, int n,
                               int T, int pass_lo, int pass_hi, double *S, double *chunks, hipStream_t s);
hipError_t launch_grad_reduce(const double *S, const double *H, const double *dlde, int B, int L, int n,
                              void *grad, int io64, hipStream_t s);
// The training step's reductions on the whole-circuit path (one <O> partial per sample) in
// one launch: E, loss, dL/dE (kept in dlde) and the gradient, bitwise as launch_ez_reduce
// followed by launch_grad_reduce.
hipError_t launch_small_reduce(const void *e_part, int r64, int B, const void *y, void *e_out, void *loss, int io64,
                               double *dlde, const double *S, const double *H, int L, int n, void *grad,
                               hipStream_t s);
// gate-by-gate comparator (hqml_gbg.hip)
hipError_t launch_gbg_zero(float2 *psi, int n, int B, hipStream_t s);
hipError_t launch_gbg_rot(int gate, float2 *psi, int n, int B, int q, const float *ang, int ang_stride,
                          hipStream_t s);
hipError_t launch_gbg_cz(float2 *psi, float2 *lam, int n, int B, int q, hipStream_t s);
hipError_t launch_gbg_cnot(float2 *psi, float2 *lam, int n, int B, int q, hipStream_t s);
hipError_t launch_gbg_expz(const float2 *psi, int n, int B, uint32_t obs, uint32_t obs_x, float *e_part,
                           hipStream_t s);
hipError_t launch_gbg_seed(const float2 *psi, float2 *lam, int n, int B, uint32_t obs, uint32_t obs_x,
                           hipStream_t s);
hipError_t launch_gbg_rot_adj(int gate, float2 *psi, float2 *lam, int n, int B, int q, const float *ang,
                              double *gpart, hipStream_t s);
hipError_t launch_gbg_grad(const double *gpart, const double *dlde, int B, int n, int n_params, float *grad,
                           hipStream_t s);
hipError_t launch_gbg_copy(const float *src, int count, float *dst, hipStream_t s);
}  // namespace hqml

namespace hqml {
// hqml_config validation and the plan it implies (HQML_OK or an hqml_status, message
// in *err).
int validate_config(const hqml_config *cfg, Plan *plan, std::string *err);

// A caller array must be device memory of `device` (or pinned host memory mapped into
// it) with at least `bytes` bytes before the end of the HIP allocation that holds it.
// HQML_OK, or HQML_ERR_ARG with a message in *err.  *base / *size (optional) receive
// that allocation's range.
int check_device_array(int device, const void *p, size_t bytes, const char *name, std::string *err,
                       const void **base = nullptr, size_t *size = nullptr);

// The message hqml_last_error(NULL) returns on this thread.
void set_thread_error(const std::string &msg);

// Observable of a configuration as the kernels take it (Z part, X part); the default
// is Z on qubit 0.
void config_observable(const hqml_config *cfg, const Plan &plan, uint32_t *z, uint32_t *x, bool *neg);
}  // namespace hqml
