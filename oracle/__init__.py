"""fp64 CPU oracle of the CSA + HCA path. Test infrastructure only (see csa_oracle)."""
