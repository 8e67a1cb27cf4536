// Internal to libpst's C ABI: the host forest handle and the thread-local
// error status shared by the host-only entry points (capi_host.cpp, plain
// C++) and the device ones (capi.cpp, HIP).
#pragma once

#include <string>

#include "host/forest.h"
#include "pst.h"

struct pst_forest {
  pst::Forest f;
};

namespace pst {

// Records `msg` as this thread's last error and returns `code`.
int fail(int code, const std::string& msg);
// Clears this thread's last error and returns PST_OK.
int ok();
// Fills the sizes of one tree.
void fill_sizes(const Tree& t, pst_tree_sizes* s);
// PST_OK, or PST_EINVAL / PST_ERANGE for a NULL forest or a bad tree index.
int check_tree(const pst_forest* forest, int32_t tree);

}  // namespace pst
