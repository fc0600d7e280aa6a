"""fp64 CPU oracle of the FASA decode step.  Test infrastructure only: the
product path never imports it."""
