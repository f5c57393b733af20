// Host-side helpers for argument validation of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe_decode.h"

namespace moe {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_F16 || dt == MOE_BF16; }

// The integer an enum argument or field holds, as the caller passed it.  A C
// caller may pass any int, and in C++ an int outside an enum's enumerators is
// not a value of that type (reading it as one is undefined), so the library
// reads the bits of every moe_dtype and moe_status it is given.
template <typename E>
inline int raw_enum(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "enums of the C ABI are int-sized");
    int v;
    __builtin_memcpy(&v, &e, sizeof v);
    return v;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// p is aligned to the size of an element of dtype dt (a valid dtype).
inline bool aligned_elem(const void *p, int dt) {
    return (reinterpret_cast<uintptr_t>(p) & (dt == MOE_F32 ? 3u : 1u)) == 0;
}

// Host checks of an RMSNorm descriptor (not null).
inline moe_status check_rmsnorm(const moe_rmsnorm *norm) {
    if (!norm || !norm->weight || !norm->normed) return MOE_EINVAL;
    const int w_dt = raw_enum(norm->dtype), n_dt = raw_enum(norm->normed_dtype);
    if (!valid_dtype(w_dt) || !valid_dtype(n_dt)) return MOE_EUNSUPPORTED;
    if (!(norm->eps >= 0.0f) || norm->eps > 3.0e38f) return MOE_EINVAL;     // NaN fails the first test
    if (!aligned_elem(norm->weight, w_dt) || !aligned_elem(norm->normed, n_dt)) return MOE_EINVAL;
    return MOE_OK;
}

// Checks one projection stack in isolation.  Returns MOE_OK or the error.
inline moe_status check_qmat(const moe_qmat *m) {
    if (!m || !m->q || !m->scales || !m->biases) return MOE_EINVAL;
    if (m->bits != 4 && m->bits != 6 && m->bits != 8) return MOE_EUNSUPPORTED;
    if (m->group_size != 64) return MOE_EUNSUPPORTED;
    if (raw_enum(m->sb_dtype) != MOE_F16 && raw_enum(m->sb_dtype) != MOE_BF16) return MOE_EUNSUPPORTED;
    if (m->n_experts < 1 || m->n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (m->rows < 64 || m->rows > MOE_MAX_DIM || m->rows % 64) return MOE_EINVAL;
    if (m->cols < 64 || m->cols > MOE_MAX_DIM || m->cols % 64) return MOE_EINVAL;
    if (!aligned16(m->q)) return MOE_EINVAL;
    if ((reinterpret_cast<uintptr_t>(m->scales) & 1u) || (reinterpret_cast<uintptr_t>(m->biases) & 1u))
        return MOE_EINVAL;
    return MOE_OK;
}

}  // namespace moe
