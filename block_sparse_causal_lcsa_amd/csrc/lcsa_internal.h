// Internal declarations shared by the host layer (lcsa_host.cpp) and the kernel files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lcsa.h"
#include "lcsa_geom.h"

namespace lcsa {

// Records a thread-local message and returns `s`.
lcsa_status fail(lcsa_status s, const char* fmt, ...)
#if defined(__GNUC__)
    __attribute__((format(printf, 2, 3)))
#endif
    ;

// Checks every field of the problem and fills the geometry. No device work.
lcsa_status validate_problem(const lcsa_problem* p, Geom* g);

// K_i for a row with n visible key blocks.
int keep_count(const lcsa_problem* p, int n);

// Checks a token tensor's base pointer and strides for [batch, heads, ntok, head_dim] access.
lcsa_status check_tensor(const char* name, const void* ptr, lcsa_strides s, const lcsa_problem* p,
                         int64_t ntok);

// check_tensor, and for a tensor the call writes: no two elements share an address (strides that
// are zero or that make rows overlap are rejected).
lcsa_status check_output_tensor(const char* name, void* ptr, lcsa_strides s, const lcsa_problem* p,
                                int64_t ntok);

// Element size in bytes of the problem's dtype.
inline int dtype_size(const lcsa_problem* p) { return p->dtype == LCSA_F32 ? 4 : 2; }

// Maps a HIP error to LCSA_ERR_HIP with its text; returns LCSA_OK for hipSuccess (0).
lcsa_status hip_status(int err, const char* what);

#if defined(__HIPCC__)
// Block means of the key tensor k (all of p's key frames, validated by the caller) written to
// out + ((b * heads + h) * out_rows + out_off + j) * head_dim for key block j (pool.hip).
lcsa_status pool_k_into(const lcsa_problem* p, const Geom& g, const void* k, lcsa_strides ks, float* out,
                        int32_t out_rows, int32_t out_off, hipStream_t s);
#endif

}  // namespace lcsa
