// The row-tile kernels of one operation, SKIPLN_ROWTILE_OP (a kOp* value):
// this file is compiled once per operation so the four sets of kernels build
// in parallel.
#include "skipln_rowtile.h"

#ifndef SKIPLN_ROWTILE_OP
#error "compile with -DSKIPLN_ROWTILE_OP=<operation>"
#endif

namespace skipln {

template <int OP>
hipError_t launch_rowtile_for(const Args& a, int dtype, int geometry, Tiling tiling, hipStream_t st) {
    using namespace rowtile;
    if (geometry < 0 || geometry >= kNumGeoms) return hipErrorInvalidValue;
    auto seq = std::make_integer_sequence<int, kNumGeoms>{};
    return dtype == 0 ? launch_geom_dispatch<float, OP>(geometry, a, tiling, st, seq)
                      : launch_geom_dispatch<_Float16, OP>(geometry, a, tiling, st, seq);
}

template <int OP>
hipError_t launch_elem_for(const Args& a, int dtype, int geometry, Tiling tiling, hipStream_t st) {
    using namespace rowtile;
    if (geometry < 0 || geometry >= kNumElemGeoms) return hipErrorInvalidValue;
    auto seq = std::make_integer_sequence<int, kNumElemGeoms>{};
    return dtype == 0 ? launch_elem_dispatch<float, OP>(geometry, a, tiling, st, seq)
                      : launch_elem_dispatch<_Float16, OP>(geometry, a, tiling, st, seq);
}

template <int OP>
hipError_t rowtile_occupancy_for(int dtype, int geometry, int form, int blocks_per_cu, int* out) {
    using namespace rowtile;
    if (geometry < 0 || geometry >= kNumGeoms) return hipErrorInvalidValue;
    auto seq = std::make_integer_sequence<int, kNumGeoms>{};
    return dtype == 0 ? occupancy_geom_dispatch<float, OP>(geometry, form, blocks_per_cu, out, seq)
                      : occupancy_geom_dispatch<_Float16, OP>(geometry, form, blocks_per_cu, out, seq);
}

template hipError_t launch_rowtile_for<SKIPLN_ROWTILE_OP>(const Args&, int, int, Tiling, hipStream_t);
template hipError_t rowtile_occupancy_for<SKIPLN_ROWTILE_OP>(int, int, int, int, int*);
template hipError_t launch_elem_for<SKIPLN_ROWTILE_OP>(const Args&, int, int, Tiling, hipStream_t);

}  // namespace skipln
