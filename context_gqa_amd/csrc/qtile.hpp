// Key range of a query tile (forward and dQ kernels): qtile_keys,
// qtile_keys_iv and qtile_full, with the rest of the index arithmetic, live
// in index.hpp, which the host index tests also compile.
#pragma once
#include "index.hpp"
